// project_mfma.hpp - the bf16 mirrored slot projection on the matrix cores
// (Technical Review §3.2, Algorithm 1 step 3): K_g = H W_K,g and V_g = H W_V,g,
// written into slot row m-1 of every KV head, plus the per-sequence boundary decision.
// A device body with caller-provided LDS, so that the projection can run as a kernel of
// its own (materialize.hip) or share one launch with the slot query (decode_attn.hip).
#pragma once

#include "masw_internal.hpp"

namespace masw {
namespace proj {

// Slot index m this call materializes for sequence b, or 0.  Only a boundary step
// t = S + W + m r with n_slots == m - 1 acts; n_slots == m means already done.
__device__ __forceinline__ int boundary_slot(const ProjectArgs& a, int b, int& bits) {
  const int t = a.seq_len[b];
  const int d = t - a.g.S - a.g.W;
  if (a.g.r < 1 || d < a.g.r || d % a.g.r) return 0;   // r = 0: no slot chain
  const int m = d / a.g.r;
  const int have = a.n_slots[b];
  if (have == m) return 0;
  if (have != m - 1) { bits |= MASW_DEV_SLOT_MISSING; return 0; }
  if (m > a.g.max_slots) { bits |= MASW_DEV_SLOT_CAPACITY; return 0; }
  return m;
}

// Prefill mode: slot index (1-based) of H row `row` = (b, slot row), or 0 if that slot
// does not exist at t = seq_len[b].  The row of slot 1 also publishes n_slots[b] = n(t).
__device__ __forceinline__ int prefill_slot(const ProjectArgs& a, int row, bool publish, int& b, int& bits) {
  b = row / a.prefill_ns;
  const int mi = row - b * a.prefill_ns;
  const int t = a.seq_len[b];
  const int d = t - a.g.S - a.g.W;
  const int n = d > 0 && a.g.r > 0 ? d / a.g.r : 0;
  if (n > a.g.max_slots || n > a.prefill_ns) {
    if (mi == 0) bits |= MASW_DEV_SLOT_CAPACITY;
    return 0;
  }
  if (publish && mi == 0) a.n_slots[b] = n;   // nothing in this launch reads n_slots
  return mi < n ? mi + 1 : 0;
}

// Rotary embedding of a slot key component ([TR] §3.2 Algorithm 1 step 6): x is the
// component, xp its pair partner, `first` whether x is the pair's first component,
// inv_freq = theta^(-2j/D) of the pair and id the slot's position id.  The angle
// (~1e5 radians at long prefixes) is formed and reduced to [-pi, pi] in fp64, then
// turned in fp32 (the reduced angle's rounding is ~2e-7 rad).
__device__ __forceinline__ float rope_turn(float x, float xp, bool first, double inv_freq, int id) {
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  const double ang = double(id) * inv_freq;
  const float red = float(ang - kTwoPi * rint(ang * (1.0 / kTwoPi)));
  float s, c;
  sincosf(red, &s, &c);
  return first ? x * c - xp * s : xp * s + x * c;
}

__device__ __forceinline__ double rope_inv_freq(int j, int D, float theta) { return pow(double(theta), -2.0 * j / D); }

// Component d of a head vector: its rotary pair partner offset (xor) and frequency index.
__device__ __forceinline__ int rope_partner_xor(int style, int D) { return style == 0 ? D / 2 : 1; }
__device__ __forceinline__ int rope_freq(int d, int style, int D) { return style == 0 ? d % (D / 2) : d / 2; }
__device__ __forceinline__ bool rope_first(int d, int style, int D) { return style == 0 ? d < D / 2 : (d & 1) == 0; }

constexpr int kCols = 64;          // output columns per work-group
constexpr int kPWaves = 4;
constexpr int kStepK = 32;         // hidden rows per MFMA step
constexpr int kPF = 4;             // steps whose weight loads a wave keeps in flight together
constexpr int kTRow = kStepK + 8;  // transposed tile row (bf16), padded: 80 bytes
// The 8-byte k-quads of transposed row n sit at quad q ^ tq_swz(n) (an even XOR keeps a
// 16-byte read of quads 2g, 2g + 1 whole): the eight rows 8 apart that one store
// instruction writes then fall on four bank groups instead of two (2-way instead of
// 4-way conflicts), and the 16-lane row reads stay conflict-free.
__device__ __forceinline__ int tq_swz(int n) { return 2 * ((n >> 4) & 3); }
constexpr int kPrefillRowGroups = 4;   // groups of 16 H rows per work-group in a prefill

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Global column of local column c (0..63) of column block nblk.  With rotate-half pairs
// at D = 128 a block takes 32 columns of a head's first half and the 32 matching ones of
// its second half, so every rotary pair lives in one work-group (lanes c and c ^ 32);
// otherwise blocks are 64 consecutive columns (at D = 64 that already pairs c, c ^ 32).
__device__ __forceinline__ int proj_col(int nblk, int c, int D, bool pair_halves) {
  if (!pair_halves || D == kCols) return nblk * kCols + c;
  const int per_head = D / kCols, head = nblk / per_head, j = nblk - head * per_head;
  return head * D + (c < 32 ? 32 * j + c : D / 2 + 32 * j + (c - 32));
}

__device__ __forceinline__ uint32_t u16_of(const u32x4_t& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Orders this wave's LDS accesses around a tile hand-over between its lanes (LDS
// executes one wave's instructions in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Grid of the projection: (N / 64 column blocks, 2 matrices, ksplits x groups of 16 RG rows of H: the
// sequences at a boundary (RG = 1), or the (sequence, slot) pairs of a prefill
// (RG = kPrefillRowGroups)).  A work-group reduces hidden rows
// [ks * k_per_split, +k_per_split) of its 64 columns; each of its 4 waves takes a
// contiguous quarter, keeps kPF steps of weight loads in flight, transposes each
// [32 k][64 n] tile through its own LDS tile and feeds, for each of its RG groups of 16
// rows, four v_mfma_f32_16x16x32_bf16 (A = H rows, zero-padded; B = the transposed
// tile), so every weight tile read serves 16 RG rows.
// Waves are summed in LDS in a fixed order; with several hidden splits the
// last-arriving work-group of the column block adds the split partials in split order
// (the ticket protocol of the decode merge), so the result is deterministic.
// LDS of one projection work-group.
template <int RG>
struct ProjectLds {
  int sm_m[16 * RG], sm_b[16 * RG];
  int sm_any, sm_last;
  __attribute__((aligned(16))) float red[kPWaves * 16 * kCols];
  __attribute__((aligned(16))) uint16_t tiles[kPWaves * kCols * kTRow];
};

// The work of work-group (nblk, which, bz) of the grid above, with its LDS in `lds`.
template <int RG>
__device__ __forceinline__ void project_mfma_body(const ProjectArgs& a, int nblk, int which, int bz, ProjectLds<RG>& lds) {
  constexpr int kRows = 16 * RG;   // rows of H per work-group
  const int bg = bz / a.ksplits, ks = bz - (bz / a.ksplits) * a.ksplits;
  const int N = a.Hkv * a.D;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int* const sm_m = lds.sm_m;
  int* const sm_b = lds.sm_b;
  int& sm_any = lds.sm_any;
  int& sm_last = lds.sm_last;
  float* const red = lds.red;
  uint16_t* const tiles = lds.tiles;

  // rows of H: sequences, or (sequence, slot) pairs in prefill mode
  const int rows = a.prefill_ns > 0 ? a.B * a.prefill_ns : a.B;
  if (tid == 0) sm_any = 0;
  __syncthreads();
  if (tid < kRows) {
    const int row = bg * kRows + tid;
    int bits = 0, m = 0, b = row;
    if (a.prefill_ns > 0) {
      if (row < rows) m = prefill_slot(a, row, nblk == 0 && which == 0 && ks == 0, b, bits);
    } else if (row < a.B) {
      m = boundary_slot(a, b, bits);
      if (nblk == 0 && which == 0 && ks == 0) a.active[b] = m;
    }
    sm_m[tid] = m;
    sm_b[tid] = b;
    if (m) atomicOr(&sm_any, 1);
    if (nblk == 0 && which == 0 && ks == 0 && bits) atomicOr(a.err, bits);
  }
  __syncthreads();
  if (!sm_any) return;

  const uint16_t* Wm = static_cast<const uint16_t*>(which ? a.w_v : a.w_k);
  const uint16_t* H = static_cast<const uint16_t*>(a.h);
  uint16_t* wt = tiles + wave * kCols * kTRow;   // this wave's transposed tile
  const int k_wave = a.k_per_split / kPWaves;                 // hidden rows of this wave
  const int kw0 = ks * a.k_per_split + wave * k_wave;
  const int n_steps = k_wave / kStepK;
  const int brow = bg * kRows + (lane & 15);   // + 16 rg
  const int col8 = lane & 7, kq = lane >> 3;   // loader: 8 lanes per 128-byte row segment
  const bool rope = a.rope_theta > 0.f;
  const bool pair_halves = rope && a.rope_style == 0 && which == 0;   // K only; V keeps whole 128-byte rows
  const int wcol = proj_col(nblk, col8 * 8, a.D, pair_halves);   // 8 columns never straddle 32

  f32x4_t acc[RG][4];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[rg][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int s0 = 0; s0 < n_steps; s0 += kPF) {
    u32x4_t wv[kPF][4];
    u32x4_t av[kPF][RG];
#pragma unroll
    for (int p = 0; p < kPF; ++p) {
      const int kk = kw0 + (s0 + p) * kStepK;
      const bool on = s0 + p < n_steps;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = kk + 4 * kq + i;
        // At a boundary every weight is read once per launch (non-temporal); a prefill's
        // row blocks share them through L2 (default policy).
        const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(Wm + size_t(k) * N + wcol);
        wv[p][i] = on && k < a.hidden ? (RG == 1 ? __builtin_nontemporal_load(wp) : *wp) : u32x4_t{0, 0, 0, 0};
      }
      const int ka = kk + (lane >> 4) * 8;
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        av[p][rg] = on && brow + 16 * rg < rows && ka < a.hidden
                        ? *reinterpret_cast<const u32x4_t*>(H + size_t(brow + 16 * rg) * a.hidden + ka)
                        : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int p = 0; p < kPF; ++p) {
      if (s0 + p >= n_steps) break;
      // transposed store: tile row n holds 32 consecutive k of column n
      wave_lds_sync();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t x0 = u16_of(wv[p][0], e) | (u16_of(wv[p][1], e) << 16);
        uint32_t x1 = u16_of(wv[p][2], e) | (u16_of(wv[p][3], e) << 16);
        *reinterpret_cast<uint2*>(wt + (col8 * 8 + e) * kTRow + 4 * (kq ^ tq_swz(col8 * 8 + e))) = make_uint2(x0, x1);
      }
      wave_lds_sync();
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int n = nt * 16 + (lane & 15);
        const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(wt + n * kTRow + 4 * ((2 * (lane >> 4)) ^ tq_swz(n)));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          acc[rg][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[p][rg]),
                                                                __builtin_bit_cast(bf16x8_t, bv), acc[rg][nt], 0, 0, 0);
      }
    }
  }

  // Rows 16 rg .. 16 rg + 15 in turn: the waves' sums meet in LDS, then each thread
  // finishes (split sum, rotation, rounding) its column of four rows.
  const int n = proj_col(nblk, tid % kCols, a.D, pair_halves);
  const int kvh = n / a.D, d = n - (n / a.D) * a.D;
  const double inv_freq = rope && which == 0 ? rope_inv_freq(rope_freq(d, a.rope_style, a.D), a.D, a.rope_theta) : 0.0;
  uint16_t* dst = static_cast<uint16_t*>(which ? a.v_slot : a.k_slot);
  constexpr int kOut = 16 * kCols / (kPWaves * kWave);   // outputs per thread
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    if (rg > 0) __syncthreads();   // the previous group's sums are read
    // D layout of a 16x16 MFMA: lane holds rows 4*(lane/16)+i of column lane%16.
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(wave * 16 + (lane >> 4) * 4 + i) * kCols + nt * 16 + (lane & 15)] = acc[rg][nt][i];
    __syncthreads();
    float s[kOut];
#pragma unroll
    for (int j = 0; j < kOut; ++j) {
      const int idx = tid + j * kPWaves * kWave;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kPWaves; ++w) v += red[w * 16 * kCols + idx];
      s[j] = v;
    }
    if constexpr (RG == 1) {
      if (a.ksplits > 1) {
        // publish this split's partial; the last split of the column block adds them up
        float* part = a.part + (size_t(bg * 2 + which) * a.ksplits) * 16 * N;
#pragma unroll
        for (int j = 0; j < kOut; ++j) {
          const int idx = tid + j * kPWaves * kWave;
          store_partial(&part[size_t(ks) * 16 * N + (idx / kCols) * N + nblk * kCols + idx % kCols], s[j]);
        }
        int32_t* cnt = a.counters + (bg * 2 + which) * (N / kCols) + nblk;
        if (!split_arrive(cnt, a.ksplits, &sm_last)) return;
#pragma unroll
        for (int j = 0; j < kOut; ++j) {
          const int idx = tid + j * kPWaves * kWave;
          const float* pp = part + (idx / kCols) * N + nblk * kCols + idx % kCols;
          float v[kMaxProjectSplits];
#pragma unroll
          for (int q = 0; q < kMaxProjectSplits; ++q) v[q] = q < a.ksplits ? load_partial(&pp[size_t(q) * 16 * N]) : 0.f;
          float t = 0.f;
#pragma unroll
          for (int q = 0; q < kMaxProjectSplits; ++q) t += v[q];   // split order; absent splits add 0
          s[j] = t;
        }
        if (tid == 0) reset_ticket(cnt);
      }
    }
    // thread tid holds local column tid % 64 (its lane) of rows tid / 64 + 4 j
#pragma unroll
    for (int j = 0; j < kOut; ++j) {
      const int idx = tid + j * kPWaves * kWave;
      const int row = rg * 16 + idx / kCols;
      const int b = sm_b[row];
      const int m = sm_m[row];
      float x = s[j];
      if (rope && which == 0) {   // uniform: every lane takes part in the exchange
        const float xp = __shfl_xor(x, a.rope_style == 0 ? 32 : 1, kWave);
        if (m > 0) x = rope_turn(x, xp, rope_first(d, a.rope_style, a.D), inv_freq, a.g.S + m * a.g.r);
      }
      if (m > 0) dst[((size_t(b) * a.Hkv + kvh) * a.g.max_slots + (m - 1)) * a.D + d] = f32_to_bf16(x);
    }
  }
}


}  // namespace proj
}  // namespace masw
