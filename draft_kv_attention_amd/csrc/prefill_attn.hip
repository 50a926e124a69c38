// prefill_attn.hip - draft prefill attention: every query of a prefix under the memory
// the draft would hold at its step (Technical Review §3.3, Algorithm 2 step 2; the
// structured mask of its Appendix C is not printed, so the reading here is that one
// pass computes what token-by-token decoding would).  Query q attends to keylist(t_q)
// (§3.1 Eq. 4): sinks, the exact window ending at t_q, slots 1..n(t_q); the raw query
// at position i has t_q = i, slot g_m's query t_q = t_m - r (§3.2 Algorithm 1 step 2).
//
// Work-group = one block of QB consecutive queries (raw positions, or slot indices) of
// one (sequence, KV head): R = QB * G <= 128 rows (query-major: row = qi * G + g).  Its
// key list is sinks ++ the raw band [max(S, t_first - W), t_last) ++ slots
// [0, n(t_last)), each row masked to its own keylist(t_q).
//
// The four waves own 32 rows each (Q in registers) and walk the key list together in
// 64-key tiles; two work-groups share a CU (64 KB of LDS each), so each SIMD holds two
// independent waves and one's softmax overlaps the other's matrix work.  The work-group
// streams the tiles through two LDS stages with asynchronous global->LDS copies (K rows
// then V rows, each row's 16-byte slots XOR-swizzled by a function of the row): one
// barrier per tile, the next tile landing while this one is computed.  Each wave
// computes, per 32-key half of the tile, on the matrix cores
//   S^T[key][row] = K[key][d] . Q^T[d][row]      (v_mfma_f32_32x32x16_bf16)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]  (V^T via ds_read_b64_tr_b16)
// with an online softmax whose reference max is only raised when a row's scores exceed
// it by more than 2^8 (the rescale of the accumulators is then rare; the result is the
// same softmax), skipping tiles none of its rows can see and masking only tiles that
// not all of its rows see whole.  P is rounded to bf16 for the second product, and the
// row sums add those same rounded weights (v_dot2_f32_bf16 against ones).
#include "masw_internal.hpp"

namespace masw {
namespace {

#ifndef MASW_PREFILL_WAVES
#define MASW_PREFILL_WAVES 4
#endif
constexpr int kPWaves = MASW_PREFILL_WAVES;
constexpr int kPThreads = kPWaves * kWave;
constexpr int kPD = 128;
constexpr int kPNB = 1;                               // row blocks of 32 per wave
constexpr int kPWaveRows = kPNB * 32;
constexpr int kPRows = kPWaves * kPWaveRows;          // rows per work-group
#ifndef MASW_PREFILL_TILE
#define MASW_PREFILL_TILE 64
#endif
constexpr int kPTile = MASW_PREFILL_TILE;             // keys per stage
constexpr int kPSub = kPTile / 32;                    // 32-key sub-tiles per stage
#ifndef MASW_PREFILL_STAGES
#define MASW_PREFILL_STAGES 2
#endif
constexpr int kPStages = MASW_PREFILL_STAGES;
constexpr int kPStageU4 = 2 * kPTile * kPD * 2 / 16;  // 16-byte words per stage (K then V)
constexpr int kPIssue = kPStageU4 / kPThreads;        // copies per thread per stage
constexpr int kPORS = kPD + 8;                        // output staging row (bf16), padded
constexpr float kLazyMax = 8.f;                       // log2 units the reference max may lag
constexpr int kPCopies = kPIssue / 2;                 // K (and V) copies per thread per stage
static_assert(kPCopies * kPThreads * 2 == kPStageU4, "the threads cover a stage");
static_assert(kPIssue * (kPStages - 2) <= 63, "s_waitcnt vmcnt holds 6 bits");
static_assert(kPStages >= 2, "two stages at least");
static_assert(kPWaves * kPWaveRows * kPORS * 2 <= kPStages * kPStageU4 * 16, "output staging fits in the stages");

typedef __bf16 pbf16x8_t __attribute__((ext_vector_type(8)));
typedef float pf32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int slots_at(int t, const MemGeom& g) {
  const int d = t - g.S - g.W;
  return d > 0 && g.r > 0 ? d / g.r : 0;
}

// Step of query index qi (0-based) of a block: raw position qi + 1, or slot qi + 1's
// t_m - r = S + W + qi * r.
__device__ __forceinline__ int query_step(bool slot_q, int qi, const MemGeom& g) {
  return slot_q ? g.S + g.W + qi * g.r : qi + 1;
}

// The work-group's key list: nsink sinks (raw rows 0..), nband band rows (raw rows
// band0..), nslot slots (slot rows 0..).
struct PKeys {
  int nsink, band0, nband, nslot;
};

// Element offset of key j's row: raw rows of the prefix ([B][p_max][Hkv][D], from the
// sequence's (row 0, kvh) base) or slot rows ([B][Hkv][max_slots][D], from its base).
__device__ __forceinline__ size_t prefill_row_off(const PKeys& kl, int j, size_t raw_stride, bool& slot) {
  slot = j >= kl.nsink + kl.nband;
  if (slot) return size_t(j - kl.nsink - kl.nband) * kPD;
  return size_t(j < kl.nsink ? j : kl.band0 + (j - kl.nsink)) * raw_stride;
}

struct PBases {
  const uint16_t* k_raw;   // prefix rows of this (sequence, KV head)
  const uint16_t* v_raw;
  const uint16_t* k_slot;  // slot rows of this (sequence, KV head)
  const uint16_t* v_slot;
  size_t raw_stride;       // elements between consecutive positions: Hkv * D
};

// Copies keys [j0, j0 + 32) into a stage: thread t moves chunk c = q * threads + t of the
// K and of the V rows, i.e. row c/16, 16-byte slot t%16, which holds the row's chunk
// (t%16) ^ tile_swz(row).  Keys past the list re-read its last key (masked).  A tile inside
// one segment takes a uniform base plus per-thread offsets; a tile across segments
// resolves each row.
__device__ __forceinline__ void prefill_issue(u32x4_t* stage, const PBases& pb, const PKeys& kl, int nk, int j0,
                                              int wave, int t, const int (&off_raw)[kPCopies], const int (&off_slot)[kPCopies]) {
  const int nraw = kl.nsink + kl.nband;
  const int j1 = j0 + kPTile;
  u32x4_t* dk = stage + wave * kWave;
  u32x4_t* dv = stage + kPStageU4 / 2 + wave * kWave;
  if (j1 <= nk && (j1 <= kl.nsink || (j0 >= kl.nsink && j1 <= nraw))) {
    // raw rows only: sinks (raw row j) or band (raw row band0 + j - nsink)
    const int r0 = j1 <= kl.nsink ? j0 : kl.band0 + (j0 - kl.nsink);
    const uint16_t* kb = pb.k_raw + size_t(r0) * pb.raw_stride;
    const uint16_t* vb = pb.v_raw + size_t(r0) * pb.raw_stride;
#pragma unroll
    for (int q = 0; q < kPCopies; ++q) {
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(kb + off_raw[q]), (lds_ptr_t)(dk + q * kPThreads), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(vb + off_raw[q]), (lds_ptr_t)(dv + q * kPThreads), 16, 0, 0);
    }
  } else if (j1 <= nk && j0 >= nraw) {
    const uint16_t* kb = pb.k_slot + size_t(j0 - nraw) * kPD;
    const uint16_t* vb = pb.v_slot + size_t(j0 - nraw) * kPD;
#pragma unroll
    for (int q = 0; q < kPCopies; ++q) {
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(kb + off_slot[q]), (lds_ptr_t)(dk + q * kPThreads), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(vb + off_slot[q]), (lds_ptr_t)(dv + q * kPThreads), 16, 0, 0);
    }
  } else {
    // the base is chosen as an integer (a select of the two pointers would be kept in
    // private memory)
    const uintptr_t kr = reinterpret_cast<uintptr_t>(pb.k_raw), ksl = reinterpret_cast<uintptr_t>(pb.k_slot);
    const uintptr_t vr = reinterpret_cast<uintptr_t>(pb.v_raw), vsl = reinterpret_cast<uintptr_t>(pb.v_slot);
#pragma unroll
    for (int q = 0; q < kPCopies; ++q) {
      const int row = (q * kPThreads + t) >> 4;
      const int chunk = (t & 15) ^ tile_swz(row);
      bool slot;
      const uintptr_t off = (prefill_row_off(kl, min(j0 + row, nk - 1), pb.raw_stride, slot) + chunk * 8) * 2;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>((slot ? ksl : kr) + off),
                                       (lds_ptr_t)(dk + q * kPThreads), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>((slot ? vsl : vr) + off),
                                       (lds_ptr_t)(dv + q * kPThreads), 16, 0, 0);
    }
  }
}

// Which keys of a tile [j0, j0 + 32) of the list the rows of one wave see: none, all
// of them (every row sees every key), or some (per-element mask).
enum TileSeen { kSeenNone = 0, kSeenAll = 1, kSeenSome = 2 };

struct WaveKeys {
  int all_sink, all_lo, all_hi, all_slot;   // seen by every row: sinks < all_sink, band raw rows
                                            // [all_lo, all_hi), slots < all_slot
  int any_sink, any_lo, any_hi, any_slot;   // seen by some row
};

__device__ __forceinline__ TileSeen tile_seen(const PKeys& kl, const WaveKeys& w, int nk, int j0) {
  const int j1 = min(j0 + kPTile, nk);
  const int nraw = kl.nsink + kl.nband;
  // one range test per segment the tile touches; [lo, hi) clipped to each segment
  bool any = false, all = j0 + kPTile <= nk;
  if (j0 < kl.nsink) {
    const int e = min(j1, kl.nsink);
    any = any || j0 < w.any_sink;
    all = all && e <= w.all_sink;
  }
  if (j1 > kl.nsink && j0 < nraw) {
    const int s = kl.band0 + (max(j0, kl.nsink) - kl.nsink), e = kl.band0 + (min(j1, nraw) - kl.nsink);
    any = any || (s < w.any_hi && e > w.any_lo);
    all = all && s >= w.all_lo && e <= w.all_hi;
  }
  if (j1 > nraw) {
    const int s = max(j0, nraw) - nraw, e = j1 - nraw;
    any = any || s < w.any_slot;
    all = all && e <= w.all_slot;
  }
  return !any ? kSeenNone : all ? kSeenAll : kSeenSome;
}

// Visible keys of one lane's row as offsets c from its first register key: sinks
// [s_lo, s_lo + s_n), band [b_lo, b_lo + b_n), slots [l_lo, l_lo + l_n) (empty when n = 0).
struct TileRanges {
  int s_lo, s_n, b_lo, b_n, l_lo, l_n;
};

// Scores of keys the row does not see become -inf: one unsigned range test per segment
// the tile touches, against the register's constant offset.
template <bool TS, bool TB, bool TL>
__device__ __forceinline__ void mask_tile(pf32x16_t (&s)[kPSub], const TileRanges& r) {
#pragma unroll
  for (int h = 0; h < kPSub; ++h)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int c = 32 * h + 8 * (v >> 2) + (v & 3);
      const bool vis = (TS && unsigned(c - r.s_lo) < unsigned(r.s_n)) || (TB && unsigned(c - r.b_lo) < unsigned(r.b_n)) ||
                       (TL && unsigned(c - r.l_lo) < unsigned(r.l_n));
      s[h][v] = vis ? s[h][v] : -INFINITY;
    }
}

// Scores of a partly seen tile that the row does not see become -inf.  The keys a row
// sees are up to three ranges of the list (its sinks, its window in the band, its
// slots); register v of sub-tile h holds key jb + c with the constant
// c = 32 h + 8 (v / 4) + v % 4.  Only the segments the tile touches (wave-uniform) are
// tested.
__device__ __forceinline__ void mask_scores(pf32x16_t (&s)[kPSub], const PKeys& kl, int j0, int half, int tq, int wlo,
                                            int nvis) {
  const int nraw = kl.nsink + kl.nband;
  const int jb = j0 + 4 * half;
  const int wl = max(wlo, kl.band0);
  const TileRanges tr{-jb, min(kl.nsink, tq), kl.nsink + (wl - kl.band0) - jb,
                      max(0, min(tq, kl.band0 + kl.nband) - wl), nraw - jb, nvis};
  const int touch = (j0 < kl.nsink ? 1 : 0) | (j0 < nraw && j0 + kPTile > kl.nsink ? 2 : 0) | (j0 + kPTile > nraw ? 4 : 0);
  switch (touch) {
    case 1: mask_tile<true, false, false>(s, tr); break;
    case 2: mask_tile<false, true, false>(s, tr); break;
    case 3: mask_tile<true, true, false>(s, tr); break;
    case 4: mask_tile<false, false, true>(s, tr); break;
    case 6: mask_tile<false, true, true>(s, tr); break;
    default: mask_tile<true, true, true>(s, tr); break;
  }
}

// Two waves per SIMD: one wave's softmax overlaps another's matrix work (with four
// waves per work-group the second wave comes from a second resident work-group).
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(const PrefillArgs a) {
  // Work-group order: slot blocks, then raw blocks, each from the last (longest key
  // list) down, with the (sequence, KV head) units innermost - the longest blocks start
  // first, and with B * Hkv a multiple of 8 each unit stays on one XCD (one L2).
  const int units = a.Hkv * a.B;
  const int unit = blockIdx.x % units, rank = blockIdx.x / units;
  const int kvh = unit % a.Hkv, b = unit / a.Hkv;
  const bool slot_q = rank < a.slot_blocks;
  const int blk = slot_q ? a.slot_blocks - 1 - rank : a.raw_blocks - 1 - (rank - a.slot_blocks);
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l32 = lane & 31, half = lane >> 5;
  const int G = a.Hq / a.Hkv;
  const MemGeom g = a.g;

  __shared__ u32x4_t pipe[kPStages][kPStageU4];

  const int P = a.seq_len[b];
  if (P == 0) return;   // empty prefix: nothing to attend
  if (P < 0 || P > a.p_max) {
    if (rank == 0 && kvh == 0 && tid == 0) atomicOr(a.err, MASW_DEV_SEQ_RANGE);
    return;
  }
  const int n_all = slots_at(P, g);
  if (n_all > g.max_slots || n_all > a.ns_max) {
    if (rank == 0 && kvh == 0 && tid == 0) atomicOr(a.err, MASW_DEV_SLOT_CAPACITY);
    return;
  }
  if (a.n_slots[b] < n_all) {
    if (rank == 0 && kvh == 0 && tid == 0) atomicOr(a.err, MASW_DEV_SLOT_MISSING);
    return;
  }
  const int q0 = blk * a.qb;
  const int nq_all = slot_q ? n_all : P;
  if (q0 >= nq_all) return;
  const int nq = min(a.qb, nq_all - q0);
  const int R = nq * G;
  const int t_first = query_step(slot_q, q0, g), t_last = query_step(slot_q, q0 + nq - 1, g);

  PKeys kl;
  kl.nsink = min(g.S, t_last);
  kl.band0 = max(g.S, t_first - g.W);
  kl.nband = max(0, t_last - kl.band0);
  kl.nslot = slots_at(t_last, g);
  const int nk = kl.nsink + kl.nband + kl.nslot;
  const int nt = (nk + kPTile - 1) / kPTile;

  PBases pb;
  pb.raw_stride = size_t(a.Hkv) * kPD;
  pb.k_raw = static_cast<const uint16_t*>(a.k) + (size_t(b) * a.p_max * a.Hkv + kvh) * kPD;
  pb.v_raw = static_cast<const uint16_t*>(a.v) + (size_t(b) * a.p_max * a.Hkv + kvh) * kPD;
  pb.k_slot = static_cast<const uint16_t*>(a.k_slot) + (size_t(b) * a.Hkv + kvh) * g.max_slots * kPD;
  pb.v_slot = static_cast<const uint16_t*>(a.v_slot) + (size_t(b) * a.Hkv + kvh) * g.max_slots * kPD;
  int off_raw[kPCopies], off_slot[kPCopies];
#pragma unroll
  for (int q = 0; q < kPCopies; ++q) {
    const int row = (q * kPThreads + tid) >> 4, chunk = (tid & 15) ^ tile_swz(row);
    off_raw[q] = row * int(pb.raw_stride) + chunk * 8;
    off_slot[q] = row * kPD + chunk * 8;
  }

  // this wave's rows [r0, r1) and the keys they see
  const int r0 = wave * kPWaveRows;
  const bool wave_on = r0 < R;
  const int r1 = min(R, r0 + kPWaveRows);
  WaveKeys wk;
  {
    const int tf = query_step(slot_q, q0 + r0 / G, g), tl = query_step(slot_q, q0 + (max(r1, r0 + 1) - 1) / G, g);
    wk.all_sink = min(g.S, tf);
    wk.all_lo = max(g.S, tl - g.W);
    wk.all_hi = tf;
    wk.all_slot = slots_at(tf, g);
    wk.any_sink = min(g.S, tl);
    wk.any_lo = max(g.S, tf - g.W);
    wk.any_hi = tl;
    wk.any_slot = slots_at(tl, g);
  }
  // per-lane row state: step, window start, visible slots (t = 0 for padding rows: no key)
  int tq[kPNB], wlo[kPNB], nvis[kPNB];
  u32x4_t bq[kPNB][8];   // Q^T operand: row r0 + rb*32 + l32, d = 16 ks + 8 half .. +7
  {
    const uint16_t* qb = static_cast<const uint16_t*>(slot_q ? a.q_slot : a.q);
    const int qstride = slot_q ? a.ns_max : a.p_max;
#pragma unroll
    for (int rb = 0; rb < kPNB; ++rb) {
      const int row = r0 + rb * 32 + l32;
      const bool ok = row < R;
      const int qi = row / G, gg = row - (row / G) * G;
      tq[rb] = ok ? query_step(slot_q, q0 + qi, g) : 0;
      wlo[rb] = max(g.S, tq[rb] - g.W);
      nvis[rb] = ok ? slots_at(tq[rb], g) : 0;
      const uint16_t* qrow = qb + ((size_t(b) * qstride + q0 + (ok ? qi : 0)) * a.Hq + size_t(kvh) * G + (ok ? gg : 0)) * kPD;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        bq[rb][ks] = ok ? *reinterpret_cast<const u32x4_t*>(qrow + ks * 16 + half * 8) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // the first tiles' copies (issued after the Q loads, so waiting for a tile also
  // covers Q)
#pragma unroll
  for (int s = 0; s < kPStages - 1; ++s)
    if (s < nt) prefill_issue(pipe[s], pb, kl, nk, s * kPTile, wave, tid, off_raw, off_slot);

  pf32x16_t o[kPNB][4];
  float m[kPNB], l[kPNB][4];   // row sums in four independent partial sums
#pragma unroll
  for (int rb = 0; rb < kPNB; ++rb) {
    m[rb] = -INFINITY;
#pragma unroll
    for (int k = 0; k < 4; ++k) l[rb][k] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[rb][db][v] = 0.f;
  }

  for (int i = 0; i < nt; ++i) {
    // tile i has landed (this thread's copies; the barrier covers everyone's), and every
    // wave is done with tile i - 1, whose stage the next copies reuse
    if (i + kPStages - 2 < nt) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPIssue * (kPStages - 2)));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (i + kPStages - 1 < nt)
      prefill_issue(pipe[(i + kPStages - 1) % kPStages], pb, kl, nk, (i + kPStages - 1) * kPTile, wave, tid, off_raw,
                    off_slot);
    if (!wave_on) continue;
    const int j0 = i * kPTile;
    const TileSeen seen = tile_seen(kl, wk, nk, j0);
    if (seen == kSeenNone) continue;

    const u32x4_t* stg = pipe[i % kPStages];
    const uint16_t* vst = reinterpret_cast<const uint16_t*>(stg + kPStageU4 / 2);
    pf32x16_t s[kPSub];
#pragma unroll
    for (int h = 0; h < kPSub; ++h) {
      u32x4_t ka[8];   // K operand (A of S^T): key 32 h + l32, d = 16 ks + 8 half .. +7
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) ka[ks] = stg[(32 * h + l32) * 16 + ((2 * ks + half) ^ tile_swz(l32))];
#pragma unroll
      for (int v = 0; v < 16; ++v) s[h][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pbf16x8_t, ka[ks]),
                                                       __builtin_bit_cast(pbf16x8_t, bq[0][ks]), s[h], 0, 0, 0);
    }
    // S^T layout: register v of sub-tile h holds key j0 + 32 h + 8*(v/4) + 4*half + v%4, row l32.
    if (seen == kSeenSome) mask_scores(s, kl, j0, half, tq[0], wlo[0], nvis[0]);
    float tmax = s[0][0];
#pragma unroll
    for (int h = 0; h < kPSub; ++h)
#pragma unroll
      for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s[h][v]);
    tmax = max_xor32(tmax);   // the row's other 32 keys sit in lane ^ 32
    const float mt = tmax * a.scale_log2;   // the tile's row max, log2 units (-inf: none seen)
    const bool grow = mt > m[0] + kLazyMax;
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m[0] - mt) : 1.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) l[0][k] *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[0][db] *= alpha;
      m[0] = grow ? mt : m[0];
    }
    const float mref = m[0] == -INFINITY ? 0.f : m[0];
    const int grp = lane >> 4, jj = lane & 15, hh = grp >> 1;
#pragma unroll
    for (int h = 0; h < kPSub; ++h) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s[h][v] = fast_exp2(fmaf(s[h][v], a.scale_log2, -mref));   // <= 2^8
      }
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        const int v0 = 8 * step;
        uint32_t pw[4];   // P^T operand: keys v0 .. v0 + 7 of this lane's row, bf16 pairs
#pragma unroll
        for (int k = 0; k < 4; ++k) pw[k] = cvt_pk_bf16(s[h][v0 + 2 * k], s[h][v0 + 2 * k + 1]);
        const u32x4_t pb4 = {pw[0], pw[1], pw[2], pw[3]};
        // the row sum adds the same bf16 weights that multiply V, two per v_dot2 (each
        // word is bit-cast from its own scalar: a bit cast of a vector element such as
        // pb4.y has compiled to a cast of element 0)
        const bf16x2_t one2 = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          l[0][step + 2 * (k >> 1)] =
              __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[k]), one2, l[0][step + 2 * (k >> 1)], false);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = db * 32 + (grp & 1) * 16 + 4 * (jj & 3);
          const int cd = d >> 3, e = d & 7;
          uint32_t w[4];
#pragma unroll
          for (int part = 0; part < 2; ++part) {
            const int key = 32 * h + 16 * step + 4 * hh + 8 * part + (jj >> 2);
            const uint16_t* src = vst + key * kPD + ((cd ^ tile_swz(key)) << 3) + e;
            const u32x2_t y = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)src));
            w[2 * part] = y.x;
            w[2 * part + 1] = y.y;
          }
          o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pbf16x8_t, u32x4_t{w[0], w[1], w[2], w[3]}),
                                                             __builtin_bit_cast(pbf16x8_t, pb4), o[0][db], 0, 0, 0);
        }
      }
    }
  }

  // Normalize and write: each wave stages its rows as bf16 in LDS (the stages are free
  // once every wave is past the loop), then stores whole 16-byte pieces of rows.
  __syncthreads();
  if (!wave_on) return;
  uint16_t* so = reinterpret_cast<uint16_t*>(&pipe[0][0]) + wave * kPWaveRows * kPORS;
#pragma unroll
  for (int rb = 0; rb < kPNB; ++rb) {
    const float lw = (l[rb][0] + l[rb][1]) + (l[rb][2] + l[rb][3]);
    const float lt = lw + __shfl_xor(lw, 32, kWave);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* dst = so + (rb * 32 + l32) * kPORS + 4 * half;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<u32x2_t*>(dst + db * 32 + 8 * g4) =
            u32x2_t{cvt_pk_bf16(o[rb][db][4 * g4] * inv, o[rb][db][4 * g4 + 1] * inv),
                    cvt_pk_bf16(o[rb][db][4 * g4 + 2] * inv, o[rb][db][4 * g4 + 3] * inv)};
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint16_t* outp = static_cast<uint16_t*>(slot_q ? a.o_slot : a.out);
  const int ostride = slot_q ? a.ns_max : a.p_max;
#pragma unroll
  for (int c = lane; c < kPWaveRows * 16; c += kWave) {
    const int row = r0 + (c >> 4), ch = c & 15;
    if (row >= r1) break;
    const int qi = row / G, gg = row - (row / G) * G;
    *reinterpret_cast<u32x4_t*>(outp + ((size_t(b) * ostride + q0 + qi) * a.Hq + size_t(kvh) * G + gg) * kPD +
                                ch * 8) = *reinterpret_cast<const u32x4_t*>(so + (c >> 4) * kPORS + ch * 8);
  }
}

}  // namespace

int launch_prefill(const PrefillArgs& a, hipStream_t s) {
  const long blocks = long(a.raw_blocks + a.slot_blocks) * a.Hkv * a.B;
  if (blocks < 1) return MASW_OK;
  if (a.qb < 1 || a.qb * (a.Hq / a.Hkv) > kPRows) return MASW_ERR_SHAPE;
  hipLaunchKernelGGL(prefill_kernel, dim3(unsigned(blocks)), dim3(kPThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? MASW_OK : MASW_ERR_LAUNCH;
}

int prefill_rows_per_block() { return kPRows; }

}  // namespace masw
