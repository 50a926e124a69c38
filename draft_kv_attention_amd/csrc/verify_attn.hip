// verify_attn.hip - verifier attention over the full cache on the matrix cores
// (Technical Review §3.3, Algorithm 2 step 5: the target checks the L_draft candidates
// in one parallel pass over its own, uncompressed KV).
//
// n_q candidate queries sit at positions t-n_q+1 .. t; query j attends to keys
// 1 .. t-n_q+1+j.  Per (sequence, KV head) the G query heads times n_q candidates form
// R = G * n_q <= 64 rows (24 for a 32/8-head layer, 48 for 64/8), in NB = ceil(R/32)
// blocks of 32 (or, for R in (32, 48], three blocks of 16: verify_stream16_kernel below).
// With 24-48 FLOP per byte the vector ALUs cannot keep pace with HBM, so both products
// run on v_mfma_f32_32x32x16_bf16:
//   S^T[key][row] = K[key][d] . Q^T[d][row]       (A = K rows, B = Q rows, both from LDS)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]   (A = V read transposed from LDS,
//                                                  B = P straight from the S^T registers)
// The transposed products make the accumulator lane own one query row, so the
// online-softmax rescale is a per-lane scalar and P never leaves registers: the S^T
// layout (lane = row, registers = keys) is the B-operand layout the second product
// needs, with its 32 keys taken in the order the registers hold them.
//
// Work-group = 4 waves over one (split, KV head, sequence): every wave streams its own
// key range through private LDS stages (verify_stream_kernel); the waves merge through
// LDS in a fixed order, and the splits are merged by a combine pass launched right after
// (verify_combine_kernel).

#include "masw_internal.hpp"

namespace masw {
namespace {

constexpr int kVWaves = 4;
constexpr int kVThreads = kVWaves * kWave;
constexpr int kD = 128;
constexpr int kMaxRows = 64;
constexpr float kVLazyMax = 8.f;   // log2 units a row's reference max may trail its true max

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int verify_chunk(int n, int n_splits, int tk) {
  int c = (n + n_splits - 1) / n_splits;
  return (c + tk - 1) / tk * tk;
}

// ---------------------------------------------------------------------------
// Every wave owns a contiguous key range of the split and
// streams it through two private LDS stages filled by asynchronous global->LDS copies,
// so the loop has no work-group barrier and two 32-key tiles (32 KB) per wave stay in
// flight while the matrix cores work on the current one.
//   stage = 16 copies of 64 lanes x 16 bytes: K rows of the tile, then V rows; row
//   `row` of the tile is 256 contiguous bytes whose 16-byte slot s holds the row's
//   chunk s ^ tile_swz(row) (the swizzle is chosen through the global address each lane
//   fetches), so neither the K-operand reads nor the transposing V-operand reads meet
//   an LDS bank conflict.
// Each wave computes all NB row blocks for its keys; the waves then merge through LDS.
// ---------------------------------------------------------------------------
constexpr int kVWaveKeys = 32;                        // keys per wave tile
constexpr int kVStageInstr = 2 * kVWaveKeys * kD * 2 / 1024;   // 16 copies of 1 KB
constexpr int kVStageU4 = kVStageInstr * kWave;       // 16-byte words per stage
constexpr int kVSplitRound = kVWaves * kVWaveKeys;    // keys per split rounding unit

__device__ __forceinline__ void verify_issue(u32x4_t* stage, const uint16_t* kbase, const uint16_t* vbase, int tile,
                                             int k1, int lane) {
  const int sub = lane >> 4, slot = lane & 15;
  if (tile + kVWaveKeys <= k1) {
    // a whole tile: one wave-uniform base plus a per-lane constant per copy
    const uint16_t* kt = kbase + size_t(tile) * kD;
    const uint16_t* vt = vbase + size_t(tile) * kD;
#pragma unroll
    for (int q = 0; q < kVWaveKeys / 4; ++q) {
      const int row = 4 * q + sub;
      const int off = row * kD + ((slot ^ tile_swz(row)) << 3);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(kt + off), (lds_ptr_t)(stage + q * kWave), 16, 0,
                                       kStreamLoadNT);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(vt + off),
                                       (lds_ptr_t)(stage + (kVWaveKeys / 4 + q) * kWave), 16, 0, kStreamLoadNT);
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < kVWaveKeys / 4; ++q) {
    const int row = 4 * q + sub;
    const int key = min(tile + row, k1 - 1);   // rows past the range re-read the last key (masked)
    const int chunk = slot ^ tile_swz(row);
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(kbase + size_t(key) * kD + chunk * 8),
                                     (lds_ptr_t)(stage + q * kWave), 16, 0, kStreamLoadNT);
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(vbase + size_t(key) * kD + chunk * 8),
                                     (lds_ptr_t)(stage + (kVWaveKeys / 4 + q) * kWave), 16, 0, kStreamLoadNT);
  }
}

// Column c of query row `row` in the wave-merge buffer: its 16-byte group (c / 4) is
// XOR-ed with the row's low 5 bits.  The rows are 512 bytes apart, so without it the
// 32 rows one accumulator store instruction writes would all land on the same four
// banks; with it they spread over all of them, and a row's pairs stay adjacent.
__device__ __forceinline__ int merge_col(int row, int c) { return c ^ ((row & 31) << 2); }

template <int NB>
__global__ __launch_bounds__(kVThreads) void verify_stream_kernel(const VerifyArgs a) {
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int G = a.Hq / a.Hkv;
  const int R = G * a.n_q;
  const int l32 = lane & 31, half = lane >> 5;

  __shared__ u32x4_t vpipe[kVWaves][2][kVStageU4];   // 128 KB; reused by the wave merge
  __shared__ float sm_ml[kVWaves][NB * 32][2];

  const int t = a.seq_len[b];
  // Q^T operand (B of S^T = K Q^T): lane holds row rb*32 + l32, d = 16 ks + 8 half .. +7,
  // in registers for every row block (with one wave per SIMD the two blocks' operands,
  // accumulators and fragments fit in its 512 registers; reading the second block's Q
  // from LDS every tile measured ~1 us slower per 70B-shaped layer).
  u32x4_t bq[NB][8];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int row = rb * 32 + l32;
    const int g = row / a.n_q, j = row - (row / a.n_q) * a.n_q;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((size_t(b) * a.n_q + (row < R ? j : 0)) * a.Hq + size_t(kvh) * G + (row < R ? g : 0)) * kD;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      bq[rb][ks] = row < R ? *reinterpret_cast<const u32x4_t*>(qrow + ks * 16 + half * 8) : u32x4_t{0, 0, 0, 0};
  }
  if (t < a.n_q || t > a.max_len) {
    if (split == 0 && kvh == 0 && threadIdx.x == 0) atomicOr(a.err, MASW_DEV_SEQ_RANGE);
    return;
  }
  const int n = t;
  const int chunk = verify_chunk(n, a.n_splits, kVSplitRound);
  const int k0 = split * chunk;
  if (k0 >= n) return;
  const int k1 = min(k0 + chunk, n);
  const int n_valid = (n + chunk - 1) / chunk;
  const int sub = chunk / kVWaves;
  const int w0 = k0 + wave * sub;
  const int w1 = min(w0 + sub, k1);
  const int nt = w0 < w1 ? (w1 - w0 + kVWaveKeys - 1) / kVWaveKeys : 0;

  // causal limit of this lane's rows: last key (0-based) query j may see
  int lim[NB];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int rho = rb * 32 + l32;
    lim[rb] = rho < R ? t - a.n_q + (rho - (rho / a.n_q) * a.n_q) : -1;
  }

  const size_t unit = size_t(b) * a.Hkv + kvh;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + unit * a.max_len * kD;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + unit * a.max_len * kD;

  f32x16_t o[NB][4];
  float m[NB], l[NB];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[rb][db][v] = 0.f;
  }

  if (nt > 0) verify_issue(vpipe[wave][0], kbase, vbase, w0, w1, lane);
  if (nt > 1) verify_issue(vpipe[wave][1], kbase, vbase, w0 + kVWaveKeys, w1, lane);
  int st = 0;
  for (int i = 0; i < nt; ++i) {
    if (i + 1 < nt) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kVStageInstr));   // only tile i+1 outstanding
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    const u32x4_t* stg = vpipe[wave][st];
    const uint16_t* vst = reinterpret_cast<const uint16_t*>(stg + kVStageU4 / 2);
    // K operand (A of S^T): key l32, d = 16 ks + 8 half .. +7
    u32x4_t ka[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ka[ks] = stg[l32 * 16 + ((2 * ks + half) ^ tile_swz(l32))];
    // V^T operand (A of O^T): lane (l32, half) holds d = 32 db + l32 for the keys
    // kb+0..3 and kb+8..11 (kb = 16 step + 4 half), the order of the S^T registers.  Two
    // transposing reads per operand: in each 16-lane group lane i, element e comes from
    // source lane 4e + i/4, element i%4, so source lane j addresses key kb + (8) + j/4,
    // columns 32 db + 16 (group%2) + 4 (j%4) .. +3 (half of one swizzled 16-byte slot).
    u32x4_t va[4][2];
    {
      const int grp = lane >> 4, j = lane & 15;
      const int hh = grp >> 1;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + (grp & 1) * 16 + 4 * (j & 3);
        const int cd = d >> 3, e = d & 7;
#pragma unroll
        for (int step = 0; step < 2; ++step) {
          uint32_t w[4];
#pragma unroll
          for (int part = 0; part < 2; ++part) {
            const int key = 16 * step + 4 * hh + 8 * part + (j >> 2);
            const uint16_t* src = vst + key * kD + ((cd ^ tile_swz(key)) << 3) + e;
            const v4i16_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)src);
            const u32x2_t y = __builtin_bit_cast(u32x2_t, x);
            w[2 * part] = y.x;
            w[2 * part + 1] = y.y;
          }
          va[db][step] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    const int tile = w0 + i * kVWaveKeys;
    if (i + 2 < nt) verify_issue(vpipe[wave][st], kbase, vbase, tile + 2 * kVWaveKeys, w1, lane);
    st ^= 1;
    const bool interior = tile + kVWaveKeys <= w1 && tile + kVWaveKeys - 1 <= t - a.n_q;

    // Score products of every row block first, the blocks' chains interleaved (each chain
    // is eight dependent MFMAs; with one wave per SIMD nothing else would fill the gaps).
    f32x16_t sacc[NB];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[rb][v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        const u32x4_t qf = bq[rb][ks];
        sacc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ka[ks]),
                                                           __builtin_bit_cast(bf16x8_t, qf), sacc[rb], 0, 0, 0);
      }

#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      f32x16_t s = sacc[rb];
      // S^T layout: register v holds key 8*(v/4) + 4*half + v%4 of the tile, row l32.
      // Tiles below every row's causal limit and inside the range need no mask.  The
      // raw scores' max is taken first (the scale is positive) and the scale goes into
      // the exponent's FMA.
      float tmax = -INFINITY;
      if (interior) {
#pragma unroll
        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s[v]);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = tile + 8 * (v >> 2) + 4 * half + (v & 3);
          s[v] = (key < w1 && key <= lim[rb]) ? s[v] : -INFINITY;
          tmax = fmaxf(tmax, s[v]);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave)) * a.scale_log2;   // log2 units; -inf: no key
      // m is the row's reference max, raised only when the tile's max passes it by more
      // than kVLazyMax: the weights stay below 2^kVLazyMax and the rescale of l and o -
      // with many rows per wave it would otherwise run on almost every tile - becomes rare.
      // The result is the same softmax: (m, l, o) stay consistent, whatever m is.
      const bool grow = tmax > m[rb] + kVLazyMax;
      if (__any(grow)) {
        const float alpha = grow ? fast_exp2(m[rb] - tmax) : 1.f;
        l[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[rb][db] *= alpha;
        m[rb] = grow ? tmax : m[rb];
      }
      const float mref = m[rb] == -INFINITY ? 0.f : m[rb];   // a row may have no key yet
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(fmaf(s[v], a.scale_log2, -mref));
        s[v] = p;
        l[rb] += p;
      }
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        const int v0 = 8 * step;
        const u32x4_t pb = {cvt_pk_bf16(s[v0 + 0], s[v0 + 1]), cvt_pk_bf16(s[v0 + 2], s[v0 + 3]),
                            cvt_pk_bf16(s[v0 + 4], s[v0 + 5]), cvt_pk_bf16(s[v0 + 6], s[v0 + 7])};
#pragma unroll
        for (int db = 0; db < 4; ++db)
          o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va[db][step]),
                                                              __builtin_bit_cast(bf16x8_t, pb), o[rb][db], 0, 0, 0);
      }
    }
  }

  // Keys of a row are split between lanes l32 and l32 + 32: total their sums.
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) l[rb] += __shfl_xor(l[rb], 32, kWave);

  // Merge the 4 waves (each holds every row over its own keys) through LDS in wave order.
  if (half == 0) {
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      sm_ml[wave][rb * 32 + l32][0] = m[rb];
      sm_ml[wave][rb * 32 + l32][1] = l[rb];
    }
  }
  __syncthreads();   // every wave is past its loop: the stages are free
  float* sm_o = reinterpret_cast<float*>(&vpipe[0][0][0]);   // [wave][NB*32 rows][128]
  static_assert(kVWaves * NB * 32 * kD * 4 <= int(sizeof(vpipe)), "wave partials fit in the stages");
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int row = rb * 32 + l32;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kVWaves; ++w) M = fmaxf(M, sm_ml[w][row][0]);
    const float wt = fast_exp2(m[rb] - (M == -INFINITY ? 0.f : M));
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        sm_o[(wave * NB * 32 + row) * kD + merge_col(row, db * 32 + 8 * (v >> 2) + 4 * half + (v & 3))] = wt * o[rb][db][v];
  }
  __syncthreads();

  // Each thread combines the waves for two adjacent columns of a row.
  uint16_t* out = static_cast<uint16_t*>(a.out);
  for (int pi = threadIdx.x; pi < R * kD / 2; pi += kVThreads) {
    const int row = 2 * pi / kD, d = 2 * pi - row * kD;
    const int g = row / a.n_q, j = row - (row / a.n_q) * a.n_q;
    const size_t prow = (size_t(b) * a.n_q + j) * a.Hq + size_t(kvh) * G + g;
    float Mr = -INFINITY;
#pragma unroll
    for (int w = 0; w < kVWaves; ++w) Mr = fmaxf(Mr, sm_ml[w][row][0]);
    const float Mrr = Mr == -INFINITY ? 0.f : Mr;
    float L = 0.f, O0 = 0.f, O1 = 0.f;
#pragma unroll
    for (int w = 0; w < kVWaves; ++w) {
      L = fmaf(fast_exp2(sm_ml[w][row][0] - Mrr), sm_ml[w][row][1], L);
      const float2 o2 = *reinterpret_cast<const float2*>(&sm_o[(w * NB * 32 + row) * kD + merge_col(row, d)]);
      O0 += o2.x;
      O1 += o2.y;
    }
    if (n_valid == 1) {
      *reinterpret_cast<uint32_t*>(out + prow * kD + d) =
          uint32_t(f32_to_bf16(O0 / L)) | (uint32_t(f32_to_bf16(O1 / L)) << 16);
    } else {
      const size_t pr = prow * a.n_splits + split;
      store_partial2(&a.part_o[pr * kD + d], O0, O1);
      if (d == 0) store_partial2(&a.part_ml[pr * 2], Mr, L);
    }
  }
}

// ---------------------------------------------------------------------------
// The same pass in row blocks of 16 on v_mfma_f32_16x16x32_bf16, for R in (32, 48]
// (64 q / 8 KV heads at 6 candidates: 48 rows).  Blocks of 32 would pad those 48 rows to
// 64; three blocks of 16 compute 48, so a 32-key tile costs three quarters of the matrix
// products and of the softmax.  Operands (lane l, group g = l / 16, i = l % 16):
//   S^T = K Q^T: A = K rows, lane holds key sigma(i) + 16 kb, d = 32 ks + 8 g .. +7;
//                B = Q rows, lane holds row 16 rb + i, the same d;
//                C: lane holds keys sigma(4 g + 0..3) + 16 kb of row 16 rb + i.
//   O^T += V^T P^T: A = V^T, lane holds d = 16 db + i for the 8 keys of its C registers
//                (two transposing reads); B = P from the C registers of both key blocks;
//                C: lane holds d = 16 db + 4 g + 0..3 of row 16 rb + i.
// sigma(m) = 8 ((m / 4) & 1) + 4 (m / 8) + m % 4 orders the keys so that one half-wave's
// transposing read covers keys {0..3, 8..11} (or {4..7, 12..15}) of each 16-key block:
// with the tile swizzle those fall on distinct banks (keys k and k + 4 would not).
// ---------------------------------------------------------------------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int v16_key_base(int g) { return 8 * (g & 1) + 4 * (g >> 1); }

template <int NB>
__global__ __launch_bounds__(kVThreads) void verify_stream16_kernel(const VerifyArgs a) {
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int G = a.Hq / a.Hkv;
  const int R = G * a.n_q;
  const int li = lane & 15, lg = lane >> 4;
  const int kbase_g = v16_key_base(lg);                     // this lane group's first key
  const int sig = v16_key_base(li >> 2) + (li & 3);         // sigma(i): key row of A lane i

  __shared__ u32x4_t vpipe[kVWaves][2][kVStageU4];   // 128 KB; reused by the wave merge
  __shared__ float sm_ml[kVWaves][NB * 16][2];

  const int t = a.seq_len[b];
  u32x4_t bq[NB][4];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int row = rb * 16 + li;
    const int g = row / a.n_q, j = row - (row / a.n_q) * a.n_q;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((size_t(b) * a.n_q + (row < R ? j : 0)) * a.Hq + size_t(kvh) * G + (row < R ? g : 0)) * kD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      bq[rb][ks] = row < R ? *reinterpret_cast<const u32x4_t*>(qrow + ks * 32 + lg * 8) : u32x4_t{0, 0, 0, 0};
  }
  if (t < a.n_q || t > a.max_len) {
    if (split == 0 && kvh == 0 && threadIdx.x == 0) atomicOr(a.err, MASW_DEV_SEQ_RANGE);
    return;
  }
  const int n = t;
  const int chunk = verify_chunk(n, a.n_splits, kVSplitRound);
  const int k0 = split * chunk;
  if (k0 >= n) return;
  const int k1 = min(k0 + chunk, n);
  const int n_valid = (n + chunk - 1) / chunk;
  const int sub = chunk / kVWaves;
  const int w0 = k0 + wave * sub;
  const int w1 = min(w0 + sub, k1);
  const int nt = w0 < w1 ? (w1 - w0 + kVWaveKeys - 1) / kVWaveKeys : 0;

  int lim[NB];   // last key (0-based) this lane's row of block rb may see
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int rho = rb * 16 + li;
    lim[rb] = rho < R ? t - a.n_q + (rho - (rho / a.n_q) * a.n_q) : -1;
  }

  const size_t unit = size_t(b) * a.Hkv + kvh;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + unit * a.max_len * kD;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + unit * a.max_len * kD;

  f32x4_t o[NB][8];
  float m[NB], l[NB];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[rb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  if (nt > 0) verify_issue(vpipe[wave][0], kbase, vbase, w0, w1, lane);
  if (nt > 1) verify_issue(vpipe[wave][1], kbase, vbase, w0 + kVWaveKeys, w1, lane);
  int st = 0;
  for (int i = 0; i < nt; ++i) {
    if (i + 1 < nt) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kVStageInstr));   // only tile i+1 outstanding
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    const u32x4_t* stg = vpipe[wave][st];
    const uint16_t* vst = reinterpret_cast<const uint16_t*>(stg + kVStageU4 / 2);
    u32x4_t ka[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = 16 * kb + sig;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ka[kb][ks] = stg[row * 16 + ((4 * ks + lg) ^ tile_swz(row))];
    }
    // V^T operand of d block db: element e of read `part` is key 16 part + kbase_g + e at
    // column 16 db + i.  In each 16-lane group, output lane i element e comes from source
    // lane 4e + i/4 element i%4, so source lane j addresses key 16 part + kbase_g + j/4,
    // columns 16 db + 4 (j%4) .. +3.
    u32x4_t va[8];
    {
      const int j = lane & 15;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int d = db * 16 + 4 * (j & 3);
        const int cd = d >> 3, e = d & 7;
        uint32_t w[4];
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const int key = 16 * part + kbase_g + (j >> 2);
          const uint16_t* src = vst + key * kD + ((cd ^ tile_swz(key)) << 3) + e;
          const v4i16_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)src);
          const u32x2_t y = __builtin_bit_cast(u32x2_t, x);
          w[2 * part] = y.x;
          w[2 * part + 1] = y.y;
        }
        va[db] = u32x4_t{w[0], w[1], w[2], w[3]};
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    const int tile = w0 + i * kVWaveKeys;
    if (i + 2 < nt) verify_issue(vpipe[wave][st], kbase, vbase, tile + 2 * kVWaveKeys, w1, lane);
    st ^= 1;
    const bool interior = tile + kVWaveKeys <= w1 && tile + kVWaveKeys - 1 <= t - a.n_q;

    // Score products of every (row block, key block), four-deep chains interleaved.
    f32x4_t sacc[NB][2];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[rb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int rb = 0; rb < NB; ++rb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sacc[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[kb][ks]),
                                                                 __builtin_bit_cast(bf16x8_t, bq[rb][ks]), sacc[rb][kb], 0, 0, 0);

#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      // register v = 4 kb + c holds key 16 kb + kbase_g + c of the tile, row 16 rb + li
      float s[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) s[v] = sacc[rb][v >> 2][v & 3];
      float tmax = -INFINITY;
      if (interior) {
#pragma unroll
        for (int v = 0; v < 8; ++v) tmax = fmaxf(tmax, s[v]);
      } else {
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int key = tile + 16 * (v >> 2) + kbase_g + (v & 3);
          s[v] = (key < w1 && key <= lim[rb]) ? s[v] : -INFINITY;
          tmax = fmaxf(tmax, s[v]);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave)) * a.scale_log2;   // log2 units; -inf: no key
      // Lazy reference max, as in the 32-row kernel: raised only when the tile's max
      // passes it by more than kVLazyMax, so the rescale of l and o stays rare.
      const bool grow = tmax > m[rb] + kVLazyMax;
      if (__any(grow)) {
        const float alpha = grow ? fast_exp2(m[rb] - tmax) : 1.f;
        l[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[rb][db] *= alpha;
        m[rb] = grow ? tmax : m[rb];
      }
      const float mref = m[rb] == -INFINITY ? 0.f : m[rb];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float p = fast_exp2(fmaf(s[v], a.scale_log2, -mref));
        s[v] = p;
        l[rb] += p;
      }
      const u32x4_t pb = {cvt_pk_bf16(s[0], s[1]), cvt_pk_bf16(s[2], s[3]), cvt_pk_bf16(s[4], s[5]),
                          cvt_pk_bf16(s[6], s[7])};
#pragma unroll
      for (int db = 0; db < 8; ++db)
        o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va[db]),
                                                            __builtin_bit_cast(bf16x8_t, pb), o[rb][db], 0, 0, 0);
    }
  }

  // Keys of a row are spread over the four lane groups: total their sums.
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    l[rb] += __shfl_xor(l[rb], 16, kWave);
    l[rb] += __shfl_xor(l[rb], 32, kWave);
  }

  if (lg == 0) {
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      sm_ml[wave][rb * 16 + li][0] = m[rb];
      sm_ml[wave][rb * 16 + li][1] = l[rb];
    }
  }
  __syncthreads();   // every wave is past its loop: the stages are free
  float* sm_o = reinterpret_cast<float*>(&vpipe[0][0][0]);   // [wave][NB*16 rows][128]
  static_assert(kVWaves * NB * 16 * kD * 4 <= int(sizeof(vpipe)), "wave partials fit in the stages");
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int row = rb * 16 + li;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kVWaves; ++w) M = fmaxf(M, sm_ml[w][row][0]);
    const float wt = fast_exp2(m[rb] - (M == -INFINITY ? 0.f : M));
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<f32x4_t*>(&sm_o[(wave * NB * 16 + row) * kD + merge_col(row, db * 16 + 4 * lg)]) = wt * o[rb][db];
  }
  __syncthreads();

  uint16_t* out = static_cast<uint16_t*>(a.out);
  for (int pi = threadIdx.x; pi < R * kD / 2; pi += kVThreads) {
    const int row = 2 * pi / kD, d = 2 * pi - row * kD;
    const int g = row / a.n_q, j = row - (row / a.n_q) * a.n_q;
    const size_t prow = (size_t(b) * a.n_q + j) * a.Hq + size_t(kvh) * G + g;
    float Mr = -INFINITY;
#pragma unroll
    for (int w = 0; w < kVWaves; ++w) Mr = fmaxf(Mr, sm_ml[w][row][0]);
    const float Mrr = Mr == -INFINITY ? 0.f : Mr;
    float L = 0.f, O0 = 0.f, O1 = 0.f;
#pragma unroll
    for (int w = 0; w < kVWaves; ++w) {
      L = fmaf(fast_exp2(sm_ml[w][row][0] - Mrr), sm_ml[w][row][1], L);
      const float2 o2 = *reinterpret_cast<const float2*>(&sm_o[(w * NB * 16 + row) * kD + merge_col(row, d)]);
      O0 += o2.x;
      O1 += o2.y;
    }
    if (n_valid == 1) {
      *reinterpret_cast<uint32_t*>(out + prow * kD + d) =
          uint32_t(f32_to_bf16(O0 / L)) | (uint32_t(f32_to_bf16(O1 / L)) << 16);
    } else {
      const size_t pr = prow * a.n_splits + split;
      store_partial2(&a.part_o[pr * kD + d], O0, O1);
      if (d == 0) store_partial2(&a.part_ml[pr * 2], Mr, L);
    }
  }
}

// Split merge of the verifier, a pass of its own after the attention kernel (the whole
// GPU combines the partials; merging them in the last work-group of each (sequence, KV
// head) left one CU pulling 128-256 KB).  64 threads combine one (query row, sequence),
// two columns each, with the 8-byte loads of a batch of kSplitBatch splits in flight,
// folded online.
constexpr int kCombRows = 4;   // query rows per work-group
__global__ __launch_bounds__(kCombRows * 64) void verify_combine_kernel(const VerifyArgs a, int tk) {
  constexpr int kSplitBatch = 8;
  const int r = blockIdx.x * kCombRows + (threadIdx.x >> 6), b = blockIdx.y;   // r = j * Hq + h
  const int dp = 2 * (threadIdx.x & 63);
  if (r >= a.n_q * a.Hq) return;
  const int t = a.seq_len[b];
  if (t < a.n_q || t > a.max_len) return;
  const int chunk = verify_chunk(t, a.n_splits, tk);
  const int nv = (t + chunk - 1) / chunk;
  if (nv == 1) return;   // written directly by the single work-group
  const size_t prow = size_t(b) * a.n_q * a.Hq + r;
  const float* ml = a.part_ml + prow * a.n_splits * 2;
  const float* po = a.part_o + prow * a.n_splits * kD + dp;
  float M = -INFINITY, L = 0.f, O0 = 0.f, O1 = 0.f;
  for (int s0 = 0; s0 < nv; s0 += kSplitBatch) {
    float2 p[kSplitBatch], v[kSplitBatch];
#pragma unroll
    for (int k = 0; k < kSplitBatch; ++k) {
      const bool in = s0 + k < nv;
      p[k] = in ? *reinterpret_cast<const float2*>(&ml[2 * (s0 + k)]) : make_float2(-INFINITY, 0.f);
      v[k] = in ? *reinterpret_cast<const float2*>(&po[size_t(s0 + k) * kD]) : make_float2(0.f, 0.f);
    }
    float mb = M;
#pragma unroll
    for (int k = 0; k < kSplitBatch; ++k) mb = fmaxf(mb, p[k].x);
    const float mbr = mb == -INFINITY ? 0.f : mb;   // splits past a row's causal limit carry -inf
    const float alpha = fast_exp2(M - mbr);
    L *= alpha;
    O0 *= alpha;
    O1 *= alpha;
#pragma unroll
    for (int k = 0; k < kSplitBatch; ++k) {
      const float w = fast_exp2(p[k].x - mbr);
      L = fmaf(w, p[k].y, L);
      O0 = fmaf(w, v[k].x, O0);
      O1 = fmaf(w, v[k].y, O1);
    }
    M = mb;
  }
  *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + prow * kD + dp) =
      uint32_t(f32_to_bf16(O0 / L)) | (uint32_t(f32_to_bf16(O1 / L)) << 16);
}

}  // namespace

int launch_verify_mfma(const VerifyArgs& a, hipStream_t s) {
  const int rows = a.Hq / a.Hkv * a.n_q;
  if (rows <= 32) {
    hipLaunchKernelGGL(verify_stream_kernel<1>, dim3(a.n_splits, a.Hkv, a.B), dim3(kVThreads), 0, s, a);
  } else if (rows <= 48) {
    hipLaunchKernelGGL(verify_stream16_kernel<3>, dim3(a.n_splits, a.Hkv, a.B), dim3(kVThreads), 0, s, a);
  } else if (rows <= kMaxRows) {
    hipLaunchKernelGGL(verify_stream_kernel<2>, dim3(a.n_splits, a.Hkv, a.B), dim3(kVThreads), 0, s, a);
  } else {
    return MASW_ERR_SHAPE;
  }
  const int tk = kVSplitRound;
  if (a.n_splits > 1)
    hipLaunchKernelGGL(verify_combine_kernel, dim3((a.n_q * a.Hq + kCombRows - 1) / kCombRows, a.B), dim3(kCombRows * 64),
                       0, s, a, tk);
  return hipGetLastError() == hipSuccess ? MASW_OK : MASW_ERR_LAUNCH;
}

}  // namespace masw
