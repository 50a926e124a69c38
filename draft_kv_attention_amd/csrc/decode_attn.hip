// decode_attn.hip - split-K decode attention over the compact draft memory.
//
// Computes Eq. 2 of the Technical Review (§2.3), softmax(scale * q K^T) V, for one
// query per (sequence, query head) over the key list of §3.1 Eq. 4
// (sinks ++ local window ++ slots), with grouped-query heads: the G = Hq/Hkv query
// heads of one KV head share every K/V row the work-group streams.
//
// Work decomposition (CDNA4, wave64):
//   grid  = (splits, Hkv, B); each work-group owns one contiguous chunk of the logical
//           key list of one (sequence, KV head); each of its 4 waves streams an equal
//           contiguous quarter of the chunk in tiles of TK keys (decode_tile_keys), two
//           tiles in flight as asynchronous global->LDS copies while it reduces the
//           previous one.
//   tiles = the logical key list is a few physical runs (sinks, the ring before and
//           after its wrap, the slots; new tokens of a fused append come from the
//           caller's buffer).  A tile inside one run is addressed from a wave-uniform
//           base plus a per-lane constant; only tiles that straddle runs, hold new
//           tokens or end the wave's range resolve every row through resolve_key().
//   wave  = 64/LPR rows of LPR lanes; a row holds one key.  bf16: 8 lanes x 32 bytes
//           per 256-byte row (D = 128), so a load instruction pair moves 8 whole rows;
//           q.k partial dots use v_dot2_f32_bf16 and are summed over the 8 lanes with
//           three DPP adds.  P.V also runs on v_dot2_f32_bf16: a lane pairs two of its
//           rows (one v_perm_b32 per dword) and P is rounded to bf16 for that product,
//           the usual flash-attention precision; the running sum l stays fp32.
//           fp32 (small models): 16 lanes per row and plain FMAs.
//   softmax is online (running max in log2 units, rescale when it grows); each wave
//   sums its row groups as a reduce-scatter and the waves merge through LDS.
//   splits merge in the same launch: every work-group stores an (max, sum, o) partial
//   and takes a ticket; the last one to arrive for its (sequence, KV head) - found with
//   an atomic ticket, reset to zero afterwards - loads the others in one round trip and
//   merges them (flash-decoding without a second kernel).
// Row addresses agree with resolve_key(), which maps the logical index to sink row
// i-1, ring row (i-S-1) mod (W+r) or slot row m-1 on the device, so no host round
// trip is needed when t changes.  With a fused append the newest n_new raw tokens are
// read straight from the caller's k_new/v_new and split 0 writes them into the memory
// (rows no other work-group of this launch reads).
#include "project_mfma.hpp"

namespace masw {
namespace {

// Keys of sequence b for this launch, or 0 when the sequence is skipped (device
// error bits are reported once per sequence when `report`).
__device__ __forceinline__ int decode_keys(const DecodeArgs& a, int t, int have, int act,
                                           KeySpan& ks, bool report) {
  if (a.active || a.gate_boundary) {  // slot query of masw_materialize_slot: gated by the boundary decision
    if (act <= 0) return 0;
    ks = key_span(t - a.back, a.g);
    ks.nslot += a.self_slot;
    return ks.total();
  }
  const int tv = t - a.back;
  int bits = 0;
  if (tv < 1 || t < a.min_t || t < a.n_new || (a.max_len > 0 && t > a.max_len)) {
    bits = MASW_DEV_SEQ_RANGE;
  } else {
    ks = key_span(tv, a.g);
    if (ks.nslot > a.g.max_slots) bits = MASW_DEV_SLOT_CAPACITY;
    else if (a.n_slots && have < ks.nslot) bits = MASW_DEV_SLOT_MISSING;
  }
  if (bits) {
    if (report) atomicOr(a.err, bits);
    return 0;
  }
  return ks.total();
}

constexpr int kWaves = kDecodeThreads / kWave;

// Keys per split: ceil(n / splits) rounded up to a multiple of kSplitRound, so that
// the waves of a work-group each take an equal contiguous run of whole 8-row groups.
// A function of (n, splits) only, so two memories with the same key list reduce in
// the same order.
constexpr int kSplitRound = 8 * kWaves;
__device__ __forceinline__ int split_chunk(int n, int n_splits) {
  int c = (n + n_splits - 1) / n_splits;
  return (c + kSplitRound - 1) / kSplitRound * kSplitRound;
}

template <typename T, int NW>
__device__ __forceinline__ float frag_dot(const uint32_t (&a)[NW], const uint32_t (&b)[NW]) {
  float acc = 0.f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < NW; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[i]),
                                            __builtin_bit_cast(bf16x2_t, b[i]), acc, false);
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) acc = fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), acc);
  }
  return acc;
}

// Element e of a lane fragment as fp32.
template <typename T, int NW>
__device__ __forceinline__ float frag_elem(const uint32_t (&w)[NW], int e) {
  if constexpr (sizeof(T) == 2) return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  else return __uint_as_float(w[e]);
}

// Fused append: copy the n_new new tokens of (b, kvh) into sink / ring rows.  An
// eviction of a token whose block has no slot yet is suppressed and reported.  Packets
// p < n_new * D / VEC each move 16 bytes of K and of V; when every packet has its own
// thread, the caller issued the loads at kernel start (pk / pv for packet threadIdx.x)
// and only the stores are left, so no load round trip sits on the work-group's path.
// No other work-group of the launch reads these rows: decode reads the new tokens from
// k_new / v_new, and the ring cells they overwrite hold tokens outside the window.
template <typename T, int D>
__device__ __forceinline__ bool append_prefetched(const DecodeArgs& a) {
  return a.n_new * (D * int(sizeof(T)) / 16) <= kDecodeThreads;
}

template <typename T, int D>
__device__ __forceinline__ size_t append_src(const DecodeArgs& a, int b, int kvh, int p) {
  constexpr int VEC = 16 / int(sizeof(T));
  constexpr int PKT = D / VEC;
  const int j = p / PKT;
  return ((size_t(b) * a.n_new + j) * a.Hkv + kvh) * D + (p - j * PKT) * VEC;
}

template <typename T, int D>
__device__ void append_rows(const DecodeArgs& a, int b, int kvh, int t, int have, bool report, u32x4_t pk,
                            u32x4_t pv) {
  if (t < a.n_new || (a.max_len > 0 && t > a.max_len)) return;   // reported by decode_keys
  constexpr int VEC = 16 / int(sizeof(T));
  constexpr int PKT = D / VEC;
  const size_t unit = size_t(b) * a.Hkv + kvh;
  const bool pre = append_prefetched<T, D>(a);
  int bits = 0;
  for (int p = threadIdx.x; p < a.n_new * PKT; p += kDecodeThreads) {
    const int j = p / PKT;
    const int d = (p - j * PKT) * VEC;
    const int i = t - a.n_new + 1 + j;
    T* dk;
    T* dv;
    size_t off;
    if (i <= a.g.S) {
      off = (unit * a.cap[0] + (i - 1)) * D + d;
      dk = static_cast<T*>(a.wk[0]);
      dv = static_cast<T*>(a.wv[0]);
    } else {
      const AppendFate f = append_fate(i, t, have, a.g);
      if (f == kAppendIllegal) bits |= MASW_DEV_PENDING_SLOT;
      if (f != kAppendWrite) continue;
      off = (unit * a.g.C + (i - a.g.S - 1) % a.g.C) * D + d;
      dk = static_cast<T*>(a.wk[1]);
      dv = static_cast<T*>(a.wv[1]);
    }
    if (!pre) {
      const size_t src = append_src<T, D>(a, b, kvh, p);
      pk = *reinterpret_cast<const u32x4_t*>(static_cast<const T*>(a.k_new) + src);
      pv = *reinterpret_cast<const u32x4_t*>(static_cast<const T*>(a.v_new) + src);
    }
    // written through (see store_out2)
    store_word2(dk + off, pk.x, pk.y);
    store_word2(dk + off + 8 / sizeof(T), pk.z, pk.w);
    store_word2(dv + off, pv.x, pv.y);
    store_word2(dv + off + 8 / sizeof(T), pv.z, pv.w);
  }
  if (bits && report) atomicOr(a.err, bits);
}

// Two adjacent outputs (d even) in one store.  The launch's few stores (outputs, the
// appended rows) are written through to memory like the partials, so the end of the
// launch finds no dirty L2 lines to write back: ~0.1 us per launch at batch 8 and at
// batch 1, measured side by side against plain stores.
template <typename T>
__device__ __forceinline__ void store_out2(T* p, float v0, float v1) {
  if constexpr (sizeof(T) == 2)
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p),
                       uint32_t(Elem<T>::from_f32(v0)) | (uint32_t(Elem<T>::from_f32(v1)) << 16), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    store_word2(p, __float_as_uint(v0), __float_as_uint(v1));
}

// ---------------------------------------------------------------------------
// Split merge
// ---------------------------------------------------------------------------
// Every work-group of a (sequence, KV head) stores its (max, sum, o) partial, waits for
// the stores and takes a ticket (split_arrive); the last arrival folds all partials.
// Each merging thread loads the partials of up to merge_batch<PER>() splits at once -
// every split of the batch-1 and batch-8 plans - so the merge costs one memory round
// trip; its own partial it takes from registers.
template <int PER>
constexpr int merge_batch() { return PER == 1 ? 32 : (PER == 2 ? 16 : 8); }

struct Partial {
  float m, l, o0, o1;
};

// Fold partials into the running (M, L, O0, O1) of one output pair, online: the batch
// max first, then every partial weighted against it (absent splits carry -inf).
template <int N>
__device__ __forceinline__ void fold_partials(const Partial (&p)[N], float& M, float& L, float& O0, float& O1) {
  float mb = M;
#pragma unroll
  for (int j = 0; j < N; ++j) mb = fmaxf(mb, p[j].m);
  const float alpha = fast_exp2(M - mb);   // 0 on the first batch (M = -inf)
  L *= alpha;
  O0 *= alpha;
  O1 *= alpha;
  M = mb;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float wt = fast_exp2(p[j].m - mb);
    L = fmaf(wt, p[j].l, L);
    O0 = fmaf(wt, p[j].o0, O0);
    O1 = fmaf(wt, p[j].o1, O1);
  }
}

// Fold the n_valid partials of the G query heads of one KV head, in split order, into
// `out` (PER output pairs per thread).  The fold order does not depend on which
// work-group merges, so the result is the same bits whichever one arrives last.
template <typename T, int D, int G, int PER>
__device__ __forceinline__ void merge_partials(const DecodeArgs& a, size_t row0, int n_valid, int own,
                                               const Partial (&mine)[PER], T* outb) {
  constexpr int NP = G * D / 2;
  constexpr int NB = merge_batch<PER>();
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int pi = threadIdx.x + k * kDecodeThreads;
    if (PER * kDecodeThreads != NP && pi >= NP) break;
    const int g = 2 * pi / D, d = 2 * pi - g * D;
    const float* pml = a.part_ml + (row0 + g) * a.n_splits * 2;
    const float* po = a.part_o + (row0 + g) * a.n_splits * D + d;
    float M = -INFINITY, L = 0.f, O0 = 0.f, O1 = 0.f;
    for (int s0 = 0; s0 < n_valid; s0 += NB) {
      float2 ml[NB], v[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int s = s0 + j;
        const bool ld = s < n_valid && s != own;
        ml[j] = ld ? load_partial2(pml + 2 * s) : make_float2(-INFINITY, 0.f);
        v[j] = ld ? load_partial2(po + size_t(s) * D) : make_float2(0.f, 0.f);
      }
      Partial p[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        p[j] = s0 + j == own ? mine[k] : Partial{ml[j].x, ml[j].y, v[j].x, v[j].y};
      fold_partials(p, M, L, O0, O1);
    }
    store_out2<T>(outb + g * D + d, O0 / L, O1 / L);
  }
}

// ---------------------------------------------------------------------------
// Row layout and reductions
// ---------------------------------------------------------------------------
// Lanes per key row: bf16 uses 8 lanes x 32 bytes (3 DPP steps per row reduction),
// fp32 16 lanes.  A wave instruction then covers 64 / LPR rows.
template <typename T> struct RowLayout { static constexpr int LPR = sizeof(T) == 2 ? 8 : 16; };

template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
  if constexpr (LPR == 16) {
    return row16_sum(v);
  } else {
    // quad xor 1, quad xor 2, then mirror inside the 8-lane half row
    return dpp_add<0x141>(dpp_add<0x4E>(dpp_add<0xB1>(v)));
  }
}

// Reduce across the 64 / LPR row groups of a wave (lanes equal modulo LPR).
template <int LPR>
__device__ __forceinline__ float groups_max(float v) {
  if constexpr (LPR == 8) v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false)));
  return rows4_max(v);
}
template <int LPR>
__device__ __forceinline__ float groups_sum(float v) {
  if constexpr (LPR == 8) v = dpp_add<0x128>(v);
  return rows4_sum(v);
}

// ---------------------------------------------------------------------------
// Tile addressing
// ---------------------------------------------------------------------------
// Where a lane's rows live, as element offsets from the sink base of K (and of V): the
// ring, slot and new-token blocks are separate allocations, so each is one 64-bit
// delta.  Keeping them as plain values (no struct or array of pointers to index) lets
// the per-row choice compile to v_cndmask instead of a table in scratch memory.
struct TileSrc {
  long dk_ring, dk_slot, dk_new, dv_ring, dv_slot, dv_new;
  long new_row;
  int t_old;
};

// Element offsets from kb0 / vb0 of the K and V rows of logical key j.
struct RowOff {
  long k, v;
};
template <int D>
__device__ __forceinline__ RowOff row_offsets(int j, const KeySpan& ks, const MemGeom& g, const TileSrc& src) {
  const KeyRef kr = resolve_key(j, ks, g);
  const bool is_new = kr.seg != 2 && kr.id > src.t_old;
  const long row = is_new ? long(kr.id - src.t_old - 1) * src.new_row : long(kr.row) * D;
  const long dk = is_new ? src.dk_new : (kr.seg == 0 ? 0L : (kr.seg == 1 ? src.dk_ring : src.dk_slot));
  const long dv = is_new ? src.dv_new : (kr.seg == 0 ? 0L : (kr.seg == 1 ? src.dv_ring : src.dv_slot));
  return RowOff{dk + row, dv + row};
}

// The runs of the logical key list that are contiguous rows of one memory block:
// keys [lo, hi) of run r sit at element offset off_k + j * D from the K sink base (V
// alike).  Run 0: sinks already in memory; 1, 2: window rows in the ring before and
// after its wrap; 3: slots.  New tokens of a fused append are in none of them.
struct KeyRuns {
  int lo0, hi0, lo1, hi1, lo2, hi2, lo3, hi3;
  long k0, v0, k1, v1, k2, v2, k3, v3;
};

template <int D>
__device__ __forceinline__ KeyRuns key_runs(const KeySpan& ks, const MemGeom& g, const TileSrc& src) {
  KeyRuns r;
  r.lo0 = 0;
  r.hi0 = min(ks.ns, src.t_old);                                      // sink ids j + 1 <= t_old
  r.k0 = 0;
  r.v0 = 0;
  const int n_old = max(0, min(ks.nl, src.t_old - ks.lo + 1));        // window rows in the ring
  const int to_wrap = g.C - ks.ring0;
  r.lo1 = ks.ns;
  r.hi1 = ks.ns + min(n_old, to_wrap);
  r.k1 = src.dk_ring + long(ks.ring0 - ks.ns) * D;
  r.v1 = src.dv_ring + long(ks.ring0 - ks.ns) * D;
  r.lo2 = ks.ns + to_wrap;
  r.hi2 = ks.ns + n_old;                                              // empty unless it wraps
  r.k2 = src.dk_ring - long(ks.ns + to_wrap) * D;
  r.v2 = src.dv_ring - long(ks.ns + to_wrap) * D;
  r.lo3 = ks.ns + ks.nl;
  r.hi3 = ks.total();
  r.k3 = src.dk_slot - long(ks.ns + ks.nl) * D;
  r.v3 = src.dv_slot - long(ks.ns + ks.nl) * D;
  return r;
}

// Issue the copies of one tile into one LDS stage of this wave: load instruction i (K
// rows, then V rows; chunk-major inside a row) writes 64 lanes x 16 bytes at stage + i
// KB, lane l at byte 16 l, so every lane later reads back exactly its own fragments.
// Row u of this lane is logical key tile + u*RPI + lgrp.  A tile inside one run (all
// values wave-uniform) takes its row addresses from one base plus a per-lane constant;
// any other tile resolves each row (rows past w1 re-read row w0 and are masked in the
// reduction).  Completion is tracked by vmcnt only.
template <typename T, int D, int U, int NW, int CH, int RPI, int TK>
__device__ __forceinline__ void issue_tile(u32x4_t* stage, int tile, int w0, int w1, int lgrp, const KeySpan& ks,
                                           const MemGeom& g, const T* kb0, const T* vb0, const TileSrc& src,
                                           const KeyRuns& runs) {
  constexpr int NC = NW / 4;
  bool fast = false;
  long bk = 0, bv = 0;
  if (tile + TK <= w1) {
    if (tile + TK <= runs.hi0) {
      fast = true; bk = runs.k0; bv = runs.v0;
    } else if (tile >= runs.lo1 && tile + TK <= runs.hi1) {
      fast = true; bk = runs.k1; bv = runs.v1;
    } else if (tile >= runs.lo2 && tile + TK <= runs.hi2) {
      fast = true; bk = runs.k2; bv = runs.v2;
    } else if (tile >= runs.lo3 && tile + TK <= runs.hi3) {
      fast = true; bk = runs.k3; bv = runs.v3;
    }
  }
  if (fast) {
    const T* kt = kb0 + bk + long(tile) * D;
    const T* vt = vb0 + bv + long(tile) * D;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ro = (u * RPI + lgrp) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(kt + ro + c * CH),
                                         (lds_ptr_t)(stage + (u * NC + c) * kWave), 16, 0, kStreamLoadNT);
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(vt + ro + c * CH),
                                         (lds_ptr_t)(stage + ((U + u) * NC + c) * kWave), 16, 0, kStreamLoadNT);
      }
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = tile + u * RPI + lgrp;
    const RowOff o = row_offsets<D>(j < w1 ? j : w0, ks, g, src);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(kb0 + o.k + c * CH),
                                       (lds_ptr_t)(stage + (u * NC + c) * kWave), 16, 0, kStreamLoadNT);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(vb0 + o.v + c * CH),
                                       (lds_ptr_t)(stage + ((U + u) * NC + c) * kWave), 16, 0, kStreamLoadNT);
    }
  }
}

// Read this lane's fragments of a tile back from its LDS stage (load instruction i of
// the copies wrote 16 bytes per lane at stage + i KB), then wait for the reads
// (lgkmcnt 0).  The reads are one asm statement: the copies fill the stage behind the
// compiler's back, the caller has waited for them (vmcnt), and the compiler must
// neither move the reads nor add waits of its own for the copies in flight.
template <int U, int NW>
__device__ __forceinline__ void read_tile_lds(uint32_t (&fk)[U][NW], uint32_t (&fv)[U][NW], const u32x4_t* stage,
                                              int lane) {
  constexpr int NC = NW / 4;
  static_assert(2 * U * NC == 8, "a stage is eight 1 KB copies: K rows, then V rows");
  const uint32_t addr = uint32_t(reinterpret_cast<uintptr_t>(stage + lane));
  u32x4_t x0, x1, x2, x3, x4, x5, x6, x7;
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\t"
      "ds_read_b128 %7, %8 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(x4), "=&v"(x5), "=&v"(x6), "=&v"(x7)
      : "v"(addr)
      : "memory");
  const u32x4_t x[8] = {x0, x1, x2, x3, x4, x5, x6, x7};
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fk[u][4 * c + i] = x[u * NC + c][i];
        fv[u][4 * c + i] = x[(U + u) * NC + c][i];
      }
}

// Online-softmax update of (m, l, acc) with one tile.
template <typename T, int G, int U, int NW, int EPL, int LPR, int RPI>
__device__ __forceinline__ void reduce_tile(const uint32_t (&fk)[U][NW], const uint32_t (&fv)[U][NW], int tile,
                                            int k1, int lgrp, float scale_log2, const uint32_t (&qw)[G][NW],
                                            float (&m)[G], float (&l)[G], float (&acc)[G][EPL]) {
  float s[U][G];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool valid = tile + u * RPI + lgrp < k1;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float d = row_sum<LPR>(frag_dot<T, NW>(qw[g], fk[u]));
      s[u][g] = valid ? d * scale_log2 : -INFINITY;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mt = s[0][g];
#pragma unroll
    for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u][g]);
    mt = groups_max<LPR>(mt);                 // finite: row 0 of the tile is valid
    const float mn = fmaxf(m[g], mt);
    if (mn != m[g]) {                         // wave-uniform: rescale only when the max grew
      const float alpha = fast_exp2(m[g] - mn); // 0 on the first tile (m = -inf)
      m[g] = mn;
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = fast_exp2(s[u][g] - mn);
      s[u][g] = p;
      l[g] += p;
    }
  }
  if constexpr (sizeof(T) == 2) {
    // P.V on v_dot2_f32_bf16: two rows of this lane at once, P rounded to bf16.
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      uint32_t pp[G];
#pragma unroll
      for (int g = 0; g < G; ++g)
        pp[g] = cvt_pk_bf16(s[u][g], s[u + 1][g]);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const uint32_t lo = __builtin_amdgcn_perm(fv[u + 1][w], fv[u][w], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(fv[u + 1][w], fv[u][w], 0x07060302u);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          acc[g][2 * w] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp[g]),
                                                          __builtin_bit_cast(bf16x2_t, lo), acc[g][2 * w], false);
          acc[g][2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp[g]),
                                                              __builtin_bit_cast(bf16x2_t, hi), acc[g][2 * w + 1], false);
        }
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(s[u][g], frag_elem<T, NW>(fv[u], e), acc[g][e]);
  }
}

// Sum the wave's row groups (lanes equal modulo LPR) of all G * EPL accumulators as a
// reduce-scatter: each step pairs lanes across one lane bit (5, 4, then 3 for LPR 8),
// and one permlane swap hands the lower half of the pair value k and the upper half
// value k + H, so each step costs one swap and one add per two values and halves what a
// lane holds.  Afterwards the lane of row group lgrp holds values k + NF * lgrp, k < NF
// (value g * EPL + e at x[k]).
template <int LPR, int G, int EPL>
__device__ __forceinline__ void groups_reduce_scatter(float (&acc)[G][EPL], int lane) {
  constexpr int NV = G * EPL;
  static_assert(NV % (64 / LPR) == 0, "every row group keeps the same number of values");
#define MASW_X(k) acc[(k) / EPL][(k) % EPL]
#pragma unroll
  for (int k = 0; k < NV / 2; ++k) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(MASW_X(k)), __float_as_uint(MASW_X(k + NV / 2)),
                                                    false, false);
    MASW_X(k) = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int k = 0; k < NV / 4; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(MASW_X(k)), __float_as_uint(MASW_X(k + NV / 4)),
                                                    false, false);
    MASW_X(k) = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (LPR == 8) {
    const bool hi = (lane & 8) != 0;
#pragma unroll
    for (int k = 0; k < NV / 8; ++k) {
      const float keep = hi ? MASW_X(k + NV / 8) : MASW_X(k), send = hi ? MASW_X(k) : MASW_X(k + NV / 8);
      MASW_X(k) = keep + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0x128, 0xf, 0xf, false));
    }
  }
#undef MASW_X
}

// LDS of one decode work-group: the tile stages of the pipeline (once a wave has left
// its loop, its own stages hold its accumulators for the merge of the waves), the
// waves' (max, sum) and the merge flag.
template <int G>
struct DecodeLds {
  u32x4_t pipe[kWaves][kPipeStages][kPipeStageInstr * kWave];
  float sm_m[kWaves][G], sm_l[kWaves][G];
  int sm_last;
};

// The work of work-group (split, kvh, b), with its LDS in `lds`.
template <typename T, int D, int G>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, const int split, const int kvh, const int b,
                                            DecodeLds<G>& lds) {
  constexpr int LPR = RowLayout<T>::LPR;
  constexpr int RPI = kWave / LPR;               // rows per wave instruction
  constexpr int EPL = D / LPR;                   // elements per lane of one row
  constexpr int NW = EPL * int(sizeof(T)) / 4;   // dwords per lane of one row
  constexpr int VEC = 16 / int(sizeof(T));       // elements per 16-byte chunk
  constexpr int CH = LPR * VEC;                  // elements between a lane's chunks
  constexpr int TK = decode_tile_keys<int(sizeof(T)), D>();   // keys per wave tile
  constexpr int U = TK / RPI;                    // rows per lane per tile
  constexpr int KI = 2 * U * (NW / 4);           // load instructions per tile
  constexpr int NP = G * D / 2;                  // output pairs of one KV head
  constexpr int PER = (NP + kDecodeThreads - 1) / kDecodeThreads;   // pairs per thread
  static_assert(U % 2 == 0, "rows are paired for the bf16 P.V dot products");
  static_assert(kSplitRound % (kWaves * RPI) == 0, "a wave's run is whole row groups");
  static_assert(KI == kPipeStageInstr, "a stage holds exactly one tile");
  static_assert(kPipeStages == 2, "the wait below assumes two stages");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  const int lgrp = lane / LPR;
  const int lsub = lane % LPR;

  // Start-up loads are independent of each other: issue them together.
  // (Absent per-sequence arrays read seq_len instead, so the three scalar loads go out
  // together without branches.)
  const int t = a.seq_len[b];
  const int have_raw = (a.n_slots ? a.n_slots : a.seq_len)[b];
  const int act_raw = (a.active ? a.active : a.seq_len)[b];
  const int have = a.n_slots ? have_raw : 0;
  const int act = a.active ? act_raw : (a.gate_boundary ? pending_slot(t, have, a.g) : 1);
  uint32_t qw[G][NW];
  const T* qb = static_cast<const T*>(a.q) + size_t(b) * a.qo_stride + size_t(kvh) * G * D + lsub * VEC;
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < NW / 4; ++c) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qb + g * D + c * CH);
      qw[g][4 * c] = x.x; qw[g][4 * c + 1] = x.y; qw[g][4 * c + 2] = x.z; qw[g][4 * c + 3] = x.w;
    }

  // Split 0 of every (sequence, KV head) also appends the new tokens: loads now, stores
  // after its share of the keys.
  const bool appender = a.n_new > 0 && split == 0;
  u32x4_t apk = {0, 0, 0, 0}, apv = {0, 0, 0, 0};
  if (appender && append_prefetched<T, D>(a) && int(threadIdx.x) < a.n_new * (D * int(sizeof(T)) / 16)) {
    const size_t src = append_src<T, D>(a, b, kvh, threadIdx.x);
    apk = *reinterpret_cast<const u32x4_t*>(static_cast<const T*>(a.k_new) + src);
    apv = *reinterpret_cast<const u32x4_t*>(static_cast<const T*>(a.v_new) + src);
  }

  KeySpan ks;
  const int n = decode_keys(a, t, have, act, ks, split == 0 && kvh == 0 && threadIdx.x == 0);
  if (n == 0) {
    if (appender) append_rows<T, D>(a, b, kvh, t, have, kvh == 0, apk, apv);
    return;
  }
  const int chunk = __builtin_amdgcn_readfirstlane(split_chunk(n, a.n_splits));
  const int k0 = split * chunk;
  if (k0 >= n) return;
  const int k1 = __builtin_amdgcn_readfirstlane(min(k0 + chunk, n));
  const int n_valid = (n + chunk - 1) / chunk;

  // Block bases of this (sequence, KV head): wave-uniform, so every offset between them
  // stays in scalar registers; each lane adds its own column offset lsub * VEC.
  const size_t unit = size_t(b) * a.Hkv + kvh;
  const T* ku0 = static_cast<const T*>(a.k[0]) + unit * a.cap[0] * D;
  const T* ku1 = static_cast<const T*>(a.k[1]) + unit * a.cap[1] * D;
  const T* ku2 = static_cast<const T*>(a.k[2]) + unit * a.cap[2] * D;
  const T* vu0 = static_cast<const T*>(a.v[0]) + unit * a.cap[0] * D;
  const T* vu1 = static_cast<const T*>(a.v[1]) + unit * a.cap[1] * D;
  const T* vu2 = static_cast<const T*>(a.v[2]) + unit * a.cap[2] * D;
  const int t_old = t - a.n_new;   // positions above this come from k_new / v_new
  const size_t new_row = size_t(a.Hkv) * D;
  const T* knu = a.n_new ? static_cast<const T*>(a.k_new) + (size_t(b) * a.n_new * a.Hkv + kvh) * D : ku0;
  const T* vnu = a.n_new ? static_cast<const T*>(a.v_new) + (size_t(b) * a.n_new * a.Hkv + kvh) * D : vu0;
  const T* kb0 = ku0 + lsub * VEC;
  const T* vb0 = vu0 + lsub * VEC;

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const TileSrc src{long(ku1 - ku0), long(ku2 - ku0), long(knu - ku0), long(vu1 - vu0), long(vu2 - vu0),
                    long(vnu - vu0), long(new_row), t_old};
  const KeyRuns runs = key_runs<D>(ks, a.g, src);
  // LDS: the tile stages of the pipeline; once a wave has left its loop its own stages
  // hold its (g, d) accumulators for the merge of the waves.
  constexpr int WAVE_O = kPipeStages * KI * kWave * 4;   // floats per wave
  static_assert(G * D <= WAVE_O, "a wave's stages hold its accumulators");
  auto& pipe = lds.pipe;
  float* const sm_o = reinterpret_cast<float*>(&pipe[0][0][0]);

  // Wave w streams keys [w0, w1) of the chunk, one tile at a time (the last one ragged).
  // Tile i sits in stage i mod 2.  Before tile i is read, s_waitcnt leaves only the
  // copies of tile i + 1 outstanding (copies complete in issue order); once its
  // fragments are in registers (lgkmcnt 0) the stage is refilled with tile i + 2 and
  // tile i is reduced while the copies stream.
  const int sub = chunk / kWaves;
  const int w0 = __builtin_amdgcn_readfirstlane(k0 + wave * sub);
  const int w1 = __builtin_amdgcn_readfirstlane(min(w0 + sub, k1));
  {
    const int nt = w0 < w1 ? (w1 - w0 + TK - 1) / TK : 0;   // tiles of this wave
    // The query fragments (and the append's prefetched rows) were requested together
    // with seq_len, whose value every address below needs: wait for them here, once.
    // Without this explicit wait the compiler cannot tell inside the loop that they have
    // arrived and waits for every copy in flight (vmcnt 0) before each tile's arithmetic.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
#pragma unroll
    for (int i = 0; i < kPipeStages; ++i)
      if (i < nt) issue_tile<T, D, U, NW, CH, RPI, TK>(pipe[wave][i], w0 + i * TK, w0, w1, lgrp, ks, a.g, kb0, vb0, src, runs);
    uint32_t ka[U][NW], va[U][NW];
    int st = 0;
    for (int i = 0; i < nt; ++i) {
      if (i + 1 < nt) __builtin_amdgcn_s_waitcnt(waitcnt_vm(KI));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      read_tile_lds<U, NW>(ka, va, pipe[wave][st], lane);
      const int tile = w0 + i * TK;
      if (i + kPipeStages < nt)
        issue_tile<T, D, U, NW, CH, RPI, TK>(pipe[wave][st], tile + kPipeStages * TK, w0, w1, lgrp, ks, a.g, kb0, vb0, src,
                                             runs);
      reduce_tile<T, G, U, NW, EPL, LPR, RPI>(ka, va, tile, w1, lgrp, a.scale_log2, qw, m, l, acc);
      st ^= 1;
    }
  }

  if (appender) append_rows<T, D>(a, b, kvh, t, have, kvh == 0, apk, apv);

  // Row groups of a wave share the running max; sum their partial l and o.
#pragma unroll
  for (int g = 0; g < G; ++g) l[g] = groups_sum<LPR>(l[g]);
  groups_reduce_scatter<LPR, G, EPL>(acc, lane);
  constexpr int NF = G * EPL / (kWave / LPR);   // accumulators a lane keeps

  auto& sm_m = lds.sm_m;
  auto& sm_l = lds.sm_l;
  int& sm_last = lds.sm_last;
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) { sm_m[wave][g] = m[g]; sm_l[wave][g] = l[g]; }
  }
#pragma unroll
  for (int k = 0; k < NF; ++k) {
    const int kk = k + NF * lgrp, g = kk / EPL, e = kk % EPL;
    sm_o[wave * WAVE_O + g * D + (e / VEC) * CH + lsub * VEC + e % VEC] = acc[k / EPL][k % EPL];
  }
  __syncthreads();

  const bool merged = n_valid > 1;
  T* outb = static_cast<T*>(a.out) + size_t(b) * a.qo_stride + size_t(kvh) * G * D;
  const size_t row0 = size_t(b) * a.Hq + size_t(kvh) * G;   // partial rows of this KV head
  // Each thread combines the waves for PER pairs of adjacent outputs (d, d + 1) and, with
  // several splits, publishes that partial.
  Partial mine[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int pi = threadIdx.x + k * kDecodeThreads;
    mine[k] = Partial{-INFINITY, 0.f, 0.f, 0.f};
    if (PER * kDecodeThreads != NP && pi >= NP) break;
    const int g = 2 * pi / D, d = 2 * pi - g * D;
    float M = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][g]);
    float L = 0.f, O0 = 0.f, O1 = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fast_exp2(sm_m[w][g] - M);   // idle waves carry m = -inf -> 0
      const float2 o = *reinterpret_cast<const float2*>(&sm_o[w * WAVE_O + g * D + d]);
      L = fmaf(wt, sm_l[w][g], L);
      O0 = fmaf(wt, o.x, O0);
      O1 = fmaf(wt, o.y, O1);
    }
    mine[k] = Partial{M, L, O0, O1};
    if (!merged) {
      store_out2<T>(outb + g * D + d, O0 / L, O1 / L);
    } else {
      const size_t pr = (row0 + g) * a.n_splits + split;
      store_partial2(&a.part_o[pr * D + d], O0, O1);
      if (d == 0) store_partial2(&a.part_ml[pr * 2], M, L);
    }
  }
  if (!merged) {
    if (a.n_slots_out && kvh == 0 && threadIdx.x == 0) a.n_slots_out[b] = act;
    return;
  }
  // The last work-group of this (sequence, KV head) to arrive merges every split's
  // partial and leaves the ticket at zero for the next call.
  if (!split_arrive(&a.counters[unit], n_valid, &sm_last)) return;
  merge_partials<T, D, G, PER>(a, row0, n_valid, split, mine, outb);
  if (threadIdx.x == 0) {
    reset_ticket(&a.counters[unit]);
    if (a.n_slots_out && kvh == 0) a.n_slots_out[b] = act;
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const DecodeArgs a) {
  __shared__ DecodeLds<G> lds;
  decode_body<T, D, G>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

// One launch for a slot boundary of a bf16 layer ([TR] §3.2 Algorithm 1 steps 1-4): the
// first n_proj work-groups project the slot hidden state (K_g, V_g into slot row m-1),
// the others run the slot query over keylist(t - r) - it does not read the new slot, so
// both run side by side - each sequence gated by its own boundary decision.  Every
// work-group reads n_slots at its start; the last one to finish (a launch-wide ticket)
// publishes n_slots = m for the sequences at their boundary and resets the ticket.
// Thread b of every work-group takes sequence b's decision together with its other
// start-up loads (nothing is published before every work-group has arrived, so it is
// the decision the gates saw), and the last work-group stores it without another load.
template <int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void boundary_kernel(const BoundaryArgs a) {
  __shared__ union {
    DecodeLds<G> d;
    proj::ProjectLds<1> p;
  } lds;
  __shared__ int sm_done;
  const int id = blockIdx.x;
  const bool mine = int(threadIdx.x) < a.d.B;
  int own_t = 0, own_have = 0;
  if (mine) {
    own_t = a.d.seq_len[threadIdx.x];
    own_have = a.d.n_slots[threadIdx.x];
  }
  if (id < a.n_proj) {
    proj::project_mfma_body<1>(a.p, id % a.proj_x, (id / a.proj_x) % 2, id / (2 * a.proj_x), lds.p);
  } else {
    const int q = id - a.n_proj, ns = a.d.n_splits, hk = a.d.Hkv;
    decode_body<uint16_t, D, G>(a.d, q % ns, (q / ns) % hk, q / (ns * hk), lds.d);
  }
  __syncthreads();
  if (threadIdx.x == 0)
    sm_done = __hip_atomic_fetch_add(a.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.n_wg - 1;
  __syncthreads();
  if (!sm_done) return;
  if (mine) {
    const int m = pending_slot(own_t, own_have, a.d.g);
    if (m) a.publish[threadIdx.x] = m;
  }
  for (int b = threadIdx.x + kDecodeThreads; b < a.d.B; b += kDecodeThreads) {
    const int m = pending_slot(a.d.seq_len[b], a.d.n_slots[b], a.d.g);
    if (m) a.publish[b] = m;
  }
  if (threadIdx.x == 0) reset_ticket(a.done);
}

__global__ void keylist_kernel(const MemGeom g, const int32_t* seq_len, int back, int32_t* out,
                               int max_keys) {
  const int b = blockIdx.x;
  const int t = seq_len[b] - back;
  KeySpan ks{};
  int n = 0;
  if (t >= 1) {
    ks = key_span(t, g);
    n = ks.total();
  }
  for (int j = threadIdx.x; j < max_keys; j += blockDim.x) {
    int32_t* o = out + (size_t(b) * max_keys + j) * 3;
    if (j < n) {
      const KeyRef r = resolve_key(j, ks, g);
      o[0] = r.seg; o[1] = r.row; o[2] = r.id;
    } else {
      o[0] = -1; o[1] = -1; o[2] = -1;
    }
  }
}

template <typename T, int D, int G>
int launch_typed(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<T, D, G>), dim3(a.n_splits, a.Hkv, a.B), dim3(kDecodeThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? MASW_OK : MASW_ERR_LAUNCH;
}

template <typename T, int D>
int launch_group(const DecodeArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_typed<T, D, 1>(a, s);
    case 2: return launch_typed<T, D, 2>(a, s);
    case 3: return launch_typed<T, D, 3>(a, s);
    case 4: return launch_typed<T, D, 4>(a, s);
    case 6: return launch_typed<T, D, 6>(a, s);
    case 8: return launch_typed<T, D, 8>(a, s);
    default: return MASW_ERR_SHAPE;
  }
}

template <int D, int G>
int launch_boundary_typed(const BoundaryArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((boundary_kernel<D, G>), dim3(a.n_wg), dim3(kDecodeThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? MASW_OK : MASW_ERR_LAUNCH;
}

template <int D>
int launch_boundary_group(const BoundaryArgs& a, hipStream_t s) {
  switch (a.d.Hq / a.d.Hkv) {
    case 1: return launch_boundary_typed<D, 1>(a, s);
    case 2: return launch_boundary_typed<D, 2>(a, s);
    case 3: return launch_boundary_typed<D, 3>(a, s);
    case 4: return launch_boundary_typed<D, 4>(a, s);
    case 6: return launch_boundary_typed<D, 6>(a, s);
    case 8: return launch_boundary_typed<D, 8>(a, s);
    default: return MASW_ERR_SHAPE;
  }
}

}  // namespace

int launch_boundary(const BoundaryArgs& a, int D, hipStream_t s) {
  return D == 128 ? launch_boundary_group<128>(a, s) : launch_boundary_group<64>(a, s);
}

int launch_decode(const DecodeArgs& a, int dtype, int D, hipStream_t s) {
  if (dtype == MASW_BF16) return D == 128 ? launch_group<uint16_t, 128>(a, s) : launch_group<uint16_t, 64>(a, s);
  return D == 128 ? launch_group<float, 128>(a, s) : launch_group<float, 64>(a, s);
}

int launch_debug_keylist(const MemGeom& g, const int32_t* seq_len, int B, int back, int32_t* out,
                         int max_keys, hipStream_t s) {
  hipLaunchKernelGGL(keylist_kernel, dim3(B), dim3(256), 0, s, g, seq_len, back, out, max_keys);
  return hipGetLastError() == hipSuccess ? MASW_OK : MASW_ERR_LAUNCH;
}

}  // namespace masw
