// prefill_attn.hip - draft prefill attention: every query of a prefix under the memory
// the draft would hold at its step (Technical Review §3.3, Algorithm 2 step 2; the
// structured mask of its Appendix C is not printed, so the reading here is that one
// pass computes what token-by-token decoding would).  Query q attends to keylist(t_q)
// (§3.1 Eq. 4): sinks, the exact window ending at t_q, slots 1..n(t_q); the raw query
// at position i has t_q = i, slot g_m's query t_q = t_m - r (§3.2 Algorithm 1 step 2).
//
// Work-group = one block of QB consecutive queries (raw positions, or slot indices) of
// one (sequence, KV head): R = QB * G rows (query-major: row = qi * G + g), in NB = 2
// row blocks of 32.  Its key list is sinks ++ the raw band
// [max(S, t_first - W), t_last) ++ slots [0, n(t_last)), each row masked to its own
// keylist(t_q).  The 4 waves stream contiguous quarters of that list through private
// LDS stages filled by asynchronous global->LDS copies (same tile format as the
// verifier: 32 keys, rows swizzled by 16-byte slot), and compute on the matrix cores:
//   S^T[key][row] = K[key][d] . Q^T[d][row]      (v_mfma_f32_32x32x16_bf16)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]  (V^T via ds_read_b64_tr_b16)
// then merge through LDS in wave order and write out / o_slot (bf16).
#include "masw_internal.hpp"

namespace masw {
namespace {

constexpr int kPWaves = 4;
constexpr int kPThreads = kPWaves * kWave;
constexpr int kPD = 128;
#ifndef MASW_PREFILL_NB
#define MASW_PREFILL_NB 2
#endif
constexpr int kPNB = MASW_PREFILL_NB;        // row blocks per work-group
constexpr int kPRows = kPNB * 32;
constexpr int kPRS = 136;                    // padded LDS row of Q (bf16 elements)
constexpr int kPTile = 32;                   // keys per wave tile
constexpr int kPStageInstr = 2 * kPTile * kPD * 2 / 1024;   // 16 copies of 1 KB
constexpr int kPStageU4 = kPStageInstr * kWave;
constexpr int kAccRow = kPD + 4;             // merge buffer row (fp32), padded

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

// Key j of the block's list -> global row pointer offset: sinks and band index raw rows
// of the prefix ([B][p_max][Hkv][D]), slots index the layer's slot rows.
struct PKeys {
  int nsink, band0, nband, nslot;
};

__device__ __forceinline__ const uint16_t* prefill_row(const PrefillArgs& a, const PKeys& kl, int j, int b, int kvh,
                                                       bool v) {
  const uint16_t* raw = static_cast<const uint16_t*>(v ? a.v : a.k);
  const uint16_t* slot = static_cast<const uint16_t*>(v ? a.v_slot : a.k_slot);
  if (j < kl.nsink) return raw + ((size_t(b) * a.p_max + j) * a.Hkv + kvh) * kPD;
  j -= kl.nsink;
  if (j < kl.nband) return raw + ((size_t(b) * a.p_max + kl.band0 + j) * a.Hkv + kvh) * kPD;
  j -= kl.nband;
  return slot + ((size_t(b) * a.Hkv + kvh) * a.g.max_slots + j) * kPD;
}

__device__ __forceinline__ void prefill_issue(u32x4_t* stage, const PrefillArgs& a, const PKeys& kl, int tile, int k0,
                                              int k1, int b, int kvh, int lane) {
  const int sub = lane >> 4, slot = lane & 15;
#pragma unroll
  for (int q = 0; q < kPTile / 4; ++q) {
    const int row = 4 * q + sub;
    const int j = tile + row < k1 ? tile + row : k0;   // rows past the range re-read a valid key (masked)
    const int chunk = slot ^ (row & 15);
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(prefill_row(a, kl, j, b, kvh, false) + chunk * 8),
                                     (lds_ptr_t)(stage + q * kWave), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(prefill_row(a, kl, j, b, kvh, true) + chunk * 8),
                                     (lds_ptr_t)(stage + (kPTile / 4 + q) * kWave), 16, 0, 0);
  }
}

__global__ __launch_bounds__(kPThreads) void prefill_kernel(const PrefillArgs a) {
  // Work-group order: slot blocks, then raw blocks, each from the last (longest key
  // list) down, with the (sequence, KV head) units innermost - the longest blocks start
  // first, and with B * Hkv a multiple of 8 each unit stays on one XCD (one L2).
  const int units = a.Hkv * a.B;
  const int unit = blockIdx.x % units, rank = blockIdx.x / units;
  const int kvh = unit % a.Hkv, b = unit / a.Hkv;
  const bool slot_q = rank < a.slot_blocks;
  const int blk = slot_q ? a.slot_blocks - 1 - rank : a.raw_blocks - 1 - (rank - a.slot_blocks);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l32 = lane & 31, half = lane >> 5;
  const int G = a.Hq / a.Hkv;
  const MemGeom g = a.g;

  __shared__ u32x4_t pipe[kPWaves][2][kPStageU4];           // 128 KB
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kPRows * kPRS];
  __shared__ float sm_ml[kPWaves][kPRows][2];

  const int P = a.seq_len[b];
  if (P == 0) return;   // empty prefix: nothing to attend
  if (P < 0 || P > a.p_max) {
    if (rank == 0 && kvh == 0 && threadIdx.x == 0) atomicOr(a.err, MASW_DEV_SEQ_RANGE);
    return;
  }
  const int n_all = slots_at(P, g);
  if (n_all > g.max_slots || n_all > a.ns_max) {
    if (rank == 0 && kvh == 0 && threadIdx.x == 0) atomicOr(a.err, MASW_DEV_SLOT_CAPACITY);
    return;
  }
  if (a.n_slots[b] < n_all) {
    if (rank == 0 && kvh == 0 && threadIdx.x == 0) atomicOr(a.err, MASW_DEV_SLOT_MISSING);
    return;
  }
  const int q0 = blk * a.qb;
  const int nq_all = slot_q ? n_all : P;
  if (q0 >= nq_all) return;
  const int nq = min(a.qb, nq_all - q0);
  const int R = nq * G;
  const int t_first = query_step(slot_q, q0, g), t_last = query_step(slot_q, q0 + nq - 1, g);

  // Q rows into LDS (row = qi * G + gg; rows >= R are zero)
  {
    const uint16_t* qb = static_cast<const uint16_t*>(slot_q ? a.q_slot : a.q);
    const int qstride = slot_q ? a.ns_max : a.p_max;
    for (int c = threadIdx.x; c < kPRows * 16; c += kPThreads) {
      const int row = c >> 4, ch = c & 15;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row < R) {
        const int qi = row / G, gg = row - (row / G) * G;
        v = *reinterpret_cast<const u32x4_t*>(qb + ((size_t(b) * qstride + q0 + qi) * a.Hq + size_t(kvh) * G + gg) * kPD +
                                              ch * 8);
      }
      *reinterpret_cast<u32x4_t*>(sQ + row * kPRS + ch * 8) = v;
    }
  }

  PKeys kl;
  kl.nsink = min(g.S, t_last);
  kl.band0 = max(g.S, t_first - g.W);
  kl.nband = max(0, t_last - kl.band0);
  kl.nslot = slots_at(t_last, g);
  const int nk = kl.nsink + kl.nband + kl.nslot;

  // per-lane row state for each row block: step, window start, visible slots
  int tq[kPNB], wlo[kPNB], nvis[kPNB];
#pragma unroll
  for (int rb = 0; rb < kPNB; ++rb) {
    const int row = rb * 32 + l32;
    const int qi = row / G;
    const bool ok = row < R;
    tq[rb] = ok ? query_step(slot_q, q0 + qi, g) : 0;   // t = 0: nothing visible (padding rows)
    wlo[rb] = max(g.S, tq[rb] - g.W);
    nvis[rb] = ok ? slots_at(tq[rb], g) : 0;
  }
  // keys visible to every valid row: sinks below min(S, t_first), band rows in
  // [max(S, t_last - W), t_first), slots below n(t_first)
  const int all_sink = min(g.S, t_first);
  const int all_band_lo = max(g.S, t_last - g.W), all_band_hi = t_first;
  const int all_slot = slots_at(t_first, g);

  const int sub = (nk + kPWaves * kPTile - 1) / (kPWaves * kPTile) * kPTile;
  const int w0 = wave * sub, w1 = min(w0 + sub, nk);
  const int nt = w0 < w1 ? (w1 - w0 + kPTile - 1) / kPTile : 0;

  pf32x16_t o[kPNB][4];
  float m[kPNB], l[kPNB];
#pragma unroll
  for (int rb = 0; rb < kPNB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[rb][db][v] = 0.f;
  }
  __syncthreads();   // Q staged

  if (nt > 0) prefill_issue(pipe[wave][0], a, kl, w0, w0, w1, b, kvh, lane);
  if (nt > 1) prefill_issue(pipe[wave][1], a, kl, w0 + kPTile, w0, w1, b, kvh, lane);
  int st = 0;
  for (int i = 0; i < nt; ++i) {
    if (i + 1 < nt) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPStageInstr));   // only tile i+1 outstanding
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    const u32x4_t* stg = pipe[wave][st];
    const uint16_t* vst = reinterpret_cast<const uint16_t*>(stg + kPStageU4 / 2);
    u32x4_t ka[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ka[ks] = stg[l32 * 16 + ((2 * ks + half) ^ (l32 & 15))];
    // V^T operand via transposing reads (see verify_stream_kernel for the lane mapping)
    u32x4_t va[4][2];
    {
      const int grp = lane >> 4, j = lane & 15, hh = grp >> 1;
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
            const uint16_t* src = vst + key * kPD + ((cd ^ (key & 15)) << 3) + e;
            const u32x2_t y = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)src));
            w[2 * part] = y.x;
            w[2 * part + 1] = y.y;
          }
          va[db][step] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    const int tile = w0 + i * kPTile;
    if (i + 2 < nt) prefill_issue(pipe[wave][st], a, kl, tile + 2 * kPTile, w0, w1, b, kvh, lane);
    st ^= 1;

    // is the whole tile visible to every valid row?
    const int te = min(tile + kPTile, w1);
    bool interior;
    if (te <= kl.nsink) interior = te <= all_sink;
    else if (tile >= kl.nsink && te <= kl.nsink + kl.nband)
      interior = kl.band0 + (tile - kl.nsink) >= all_band_lo && kl.band0 + (te - kl.nsink) <= all_band_hi;
    else if (tile >= kl.nsink + kl.nband) interior = te - kl.nsink - kl.nband <= all_slot;
    else interior = false;
    interior = interior && tile + kPTile <= w1;

#pragma unroll
    for (int rb = 0; rb < kPNB; ++rb) {
      pf32x16_t s;
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4_t qf = *reinterpret_cast<const u32x4_t*>(sQ + (rb * 32 + l32) * kPRS + ks * 16 + half * 8);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pbf16x8_t, ka[ks]),
                                                    __builtin_bit_cast(pbf16x8_t, qf), s, 0, 0, 0);
      }
      // S^T layout: register v holds key 8*(v/4) + 4*half + v%4 of the tile, row l32.
      float tmax = -INFINITY;
      if (interior) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          s[v] *= a.scale_log2;
          tmax = fmaxf(tmax, s[v]);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = tile + 8 * (v >> 2) + 4 * half + (v & 3);
          bool vis;
          if (j >= w1) vis = false;
          else if (j < kl.nsink) vis = j < min(g.S, tq[rb]);
          else if (j < kl.nsink + kl.nband) {
            const int x = kl.band0 + j - kl.nsink;
            vis = x >= wlo[rb] && x < tq[rb];
          } else {
            vis = j - kl.nsink - kl.nband < nvis[rb];
          }
          const float sc = vis ? s[v] * a.scale_log2 : -INFINITY;
          s[v] = sc;
          tmax = fmaxf(tmax, sc);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
      const float mn = fmaxf(m[rb], tmax);
      const float mref = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[rb] - mref);
      if (__any(mn != m[rb])) {
        l[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[rb][db] *= alpha;
      }
      m[rb] = mn;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(s[v] - mref);
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
          o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pbf16x8_t, va[db][step]),
                                                              __builtin_bit_cast(pbf16x8_t, pb), o[rb][db], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int rb = 0; rb < kPNB; ++rb) l[rb] += __shfl_xor(l[rb], 32, kWave);
  if (half == 0) {
#pragma unroll
    for (int rb = 0; rb < kPNB; ++rb) {
      sm_ml[wave][rb * 32 + l32][0] = m[rb];
      sm_ml[wave][rb * 32 + l32][1] = l[rb];
    }
  }
  __syncthreads();   // every wave is past its loop: the stages are free
  // Merge the waves: each adds its rescaled O^T into one padded [rows][132] fp32 buffer,
  // in wave order (16-byte stores, rows 4 banks apart).
  float* acc = reinterpret_cast<float*>(&pipe[0][0][0]);
  static_assert(kPRows * kAccRow * 4 <= int(sizeof(pipe)), "merge buffer fits in the stages");
  for (int w = 0; w < kPWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rb = 0; rb < kPNB; ++rb) {
        const int row = rb * 32 + l32;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kPWaves; ++ww) M = fmaxf(M, sm_ml[ww][row][0]);
        const float wt = fast_exp2(m[rb] - (M == -INFINITY ? 0.f : M));
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            float4* dst = reinterpret_cast<float4*>(acc + row * kAccRow + db * 32 + 8 * v4 + 4 * half);
            float4 x = make_float4(wt * o[rb][db][4 * v4], wt * o[rb][db][4 * v4 + 1], wt * o[rb][db][4 * v4 + 2],
                                   wt * o[rb][db][4 * v4 + 3]);
            if (w > 0) {
              const float4 y = *dst;
              x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
            }
            *dst = x;
          }
      }
    }
    __syncthreads();
  }
  // out[row] = acc[row] / L, 8 columns (16 bytes of bf16) per thread
  uint16_t* outp = static_cast<uint16_t*>(slot_q ? a.o_slot : a.out);
  const int ostride = slot_q ? a.ns_max : a.p_max;
  for (int c = threadIdx.x; c < R * 16; c += kPThreads) {
    const int row = c >> 4, ch = c & 15;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kPWaves; ++w) M = fmaxf(M, sm_ml[w][row][0]);
    const float Mr = M == -INFINITY ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kPWaves; ++w) L = fmaf(fast_exp2(sm_ml[w][row][0] - Mr), sm_ml[w][row][1], L);
    const float inv = 1.f / L;
    const float4 x0 = *reinterpret_cast<const float4*>(acc + row * kAccRow + ch * 8);
    const float4 x1 = *reinterpret_cast<const float4*>(acc + row * kAccRow + ch * 8 + 4);
    const u32x4_t y = {cvt_pk_bf16(x0.x * inv, x0.y * inv), cvt_pk_bf16(x0.z * inv, x0.w * inv),
                       cvt_pk_bf16(x1.x * inv, x1.y * inv), cvt_pk_bf16(x1.z * inv, x1.w * inv)};
    const int qi = row / G, gg = row - (row / G) * G;
    *reinterpret_cast<u32x4_t*>(outp + ((size_t(b) * ostride + q0 + qi) * a.Hq + size_t(kvh) * G + gg) * kPD +
                                ch * 8) = y;
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
