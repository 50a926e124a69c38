// decode_attn.hip - split-K decode attention over the compact draft memory.
//
// Computes Eq. 2 of the Technical Review (§2.3), softmax(scale * q K^T) V, for one
// query per (sequence, query head) over the key list of §3.1 Eq. 4
// (sinks ++ local window ++ slots), with grouped-query heads: the G = Hq/Hkv query
// heads of one KV head share every K/V row the work-group streams.
//
// Work decomposition (CDNA4, wave64):
//   grid  = (splits, Hkv, B); each work-group owns one contiguous chunk of the logical
//           key list of one (sequence, KV head) and 4 waves stride over it in tiles of
//           32 keys.
//   wave  = 4 rows of 16 lanes; a row holds one key: each lane loads D/16 elements of
//           K and of V (16 B for bf16 D=128), so one load instruction moves 4 whole
//           256-byte rows (coalesced).  q.k partial dots use v_dot2_f32_bf16 and are
//           summed over the 16 lanes with DPP row rotations.
//   softmax is online (running max in log2 units, rescale per tile); waves merge
//   through LDS, splits through a second small kernel (flash-decoding).
// Every key row is located through resolve_key(), which maps the logical index to
// sink row i-1, ring row (i-S-1) mod (W+r) or slot row m-1 on the device, so no host
// round trip is needed when t changes.
#include "masw_internal.hpp"

namespace masw {
namespace {

// Keys of sequence b for this launch, or 0 when the sequence is skipped (device
// error bits are reported once per sequence when `report`).
__device__ __forceinline__ int decode_keys(const DecodeArgs& a, int b, KeySpan& ks, bool report) {
  const int t = a.seq_len[b];
  if (a.active) {  // slot query of masw_materialize_slot: gated by the boundary decision
    if (a.active[b] <= 0) return 0;
    ks = key_span(t - a.back, a.g);
    ks.nslot += a.self_slot;
    return ks.total();
  }
  const int tv = t - a.back;
  int bits = 0;
  if (tv < 1 || (a.max_len > 0 && t > a.max_len)) {
    bits = MASW_DEV_SEQ_RANGE;
  } else {
    ks = key_span(tv, a.g);
    if (ks.nslot > a.g.max_slots) bits = MASW_DEV_SLOT_CAPACITY;
    else if (a.n_slots && a.n_slots[b] < ks.nslot) bits = MASW_DEV_SLOT_MISSING;
  }
  if (bits) {
    if (report) atomicOr(a.err, bits);
    return 0;
  }
  return ks.total();
}

// Keys per split: ceil(n / splits) rounded up to whole tiles.  A function of (n, splits)
// only, so two memories with the same key list reduce in the same order.
__device__ __forceinline__ int split_chunk(int n, int n_splits) {
  int c = (n + n_splits - 1) / n_splits;
  return (c + kDecodeTileKeys - 1) / kDecodeTileKeys * kDecodeTileKeys;
}

template <int NW>
__device__ __forceinline__ void load_frag(uint32_t (&w)[NW], const void* p) {
  if constexpr (NW == 2) {
    uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x; w[1] = x.y;
  } else if constexpr (NW == 4) {
    uint4 x = *reinterpret_cast<const uint4*>(p);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else {
    static_assert(NW == 8, "fragment size");
    uint4 x = reinterpret_cast<const uint4*>(p)[0];
    uint4 y = reinterpret_cast<const uint4*>(p)[1];
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    w[4] = y.x; w[5] = y.y; w[6] = y.z; w[7] = y.w;
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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

template <typename T, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const DecodeArgs a) {
  constexpr int EPL = D / 16;                    // elements per lane of one row
  constexpr int NW = EPL * int(sizeof(T)) / 4;   // dwords per lane of one row
  constexpr int U = kDecodeTileKeys / 4;         // rows per lane per tile
  constexpr int NWAVES = kDecodeThreads / kWave;

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int lrow = lane >> 4;
  const int l16 = lane & 15;

  KeySpan ks;
  const int n = decode_keys(a, b, ks, split == 0 && kvh == 0 && threadIdx.x == 0);
  if (n == 0) return;
  const int chunk = split_chunk(n, a.n_splits);
  const int k0 = split * chunk;
  if (k0 >= n) return;
  const int k1 = min(k0 + chunk, n);

  const size_t unit = size_t(b) * a.Hkv + kvh;
  const T* kb0 = static_cast<const T*>(a.k[0]) + unit * a.cap[0] * D + l16 * EPL;
  const T* kb1 = static_cast<const T*>(a.k[1]) + unit * a.cap[1] * D + l16 * EPL;
  const T* kb2 = static_cast<const T*>(a.k[2]) + unit * a.cap[2] * D + l16 * EPL;
  const T* vb0 = static_cast<const T*>(a.v[0]) + unit * a.cap[0] * D + l16 * EPL;
  const T* vb1 = static_cast<const T*>(a.v[1]) + unit * a.cap[1] * D + l16 * EPL;
  const T* vb2 = static_cast<const T*>(a.v[2]) + unit * a.cap[2] * D + l16 * EPL;

  uint32_t qw[G][NW];
#pragma unroll
  for (int g = 0; g < G; ++g)
    load_frag<NW>(qw[g], static_cast<const T*>(a.q) + (size_t(b) * a.Hq + kvh * G + g) * D + l16 * EPL);

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  for (int tile = k0 + wave * kDecodeTileKeys; tile < k1; tile += NWAVES * kDecodeTileKeys) {
    uint32_t kw[U][NW], vw[U][NW];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = tile + u * 4 + lrow;
      valid[u] = j < k1;
      const KeyRef kr = resolve_key(valid[u] ? j : k0, ks, a.g);
      const size_t off = size_t(kr.row) * D;
      const T* kp = kr.seg == 0 ? kb0 : (kr.seg == 1 ? kb1 : kb2);
      const T* vp = kr.seg == 0 ? vb0 : (kr.seg == 1 ? vb1 : vb2);
      load_frag<NW>(kw[u], kp + off);
      load_frag<NW>(vw[u], vp + off);
    }
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float d = row16_sum(frag_dot<T, NW>(qw[g], kw[u]));
        s[u][g] = valid[u] ? d * a.scale_log2 : -INFINITY;
      }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mt = s[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u][g]);
      mt = rows4_max(mt);                       // finite: row 0 of the tile is valid
      const float mn = fmaxf(m[g], mt);
      const float alpha = fast_exp2(m[g] - mn); // 0 on the first tile (m = -inf)
      m[g] = mn;
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = fast_exp2(s[u][g] - mn);
        l[g] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p, frag_elem<T, NW>(vw[u], e), acc[g][e]);
      }
    }
  }

  // Rows of a wave share the running max; sum their partial l and o.
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = rows4_sum(l[g]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = rows4_sum(acc[g][e]);
  }

  __shared__ float sm_m[NWAVES][G], sm_l[NWAVES][G];
  __shared__ float sm_o[NWAVES][G][D];
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) { sm_m[wave][g] = m[g]; sm_l[wave][g] = l[g]; }
  }
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wave][g][l16 * EPL + e] = acc[g][e];
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
    const int g = idx / D, d = idx - (idx / D) * D;
    float M = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) M = fmaxf(M, sm_m[w][g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
      const float wt = fast_exp2(sm_m[w][g] - M);   // idle waves carry m = -inf -> 0
      L = fmaf(wt, sm_l[w][g], L);
      O = fmaf(wt, sm_o[w][g][d], O);
    }
    const size_t row = size_t(b) * a.Hq + kvh * G + g;
    if (a.n_splits == 1) {
      static_cast<T*>(a.out)[row * D + d] = Elem<T>::from_f32(O / L);
    } else {
      const size_t pr = row * a.n_splits + split;
      a.part_o[pr * D + d] = O;
      if (d == 0) { a.part_ml[pr * 2] = M; a.part_ml[pr * 2 + 1] = L; }
    }
  }
  if (a.n_splits == 1 && a.n_slots_out && kvh == 0 && threadIdx.x == 0) a.n_slots_out[b] = a.active[b];
}

// Merge the per-split (max, sum, o) partials of one (sequence, query head).
template <typename T, int D>
__global__ __launch_bounds__(D) void combine_kernel(const DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  KeySpan ks;
  const int n = decode_keys(a, b, ks, false);
  if (n == 0) return;
  const int chunk = split_chunk(n, a.n_splits);
  const int nv = (n + chunk - 1) / chunk;
  const size_t row = size_t(b) * a.Hq + h;
  const float* ml = a.part_ml + row * a.n_splits * 2;
  const float* po = a.part_o + row * a.n_splits * D + d;
  float M = -INFINITY;
  for (int s = 0; s < nv; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f, O = 0.f;
  for (int s = 0; s < nv; ++s) {
    const float wt = fast_exp2(ml[2 * s] - M);
    L = fmaf(wt, ml[2 * s + 1], L);
    O = fmaf(wt, po[size_t(s) * D], O);
  }
  static_cast<T*>(a.out)[row * D + d] = Elem<T>::from_f32(O / L);
  if (a.n_slots_out && h == 0 && d == 0) a.n_slots_out[b] = a.active[b];
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
  if (a.n_splits > 1)
    hipLaunchKernelGGL((combine_kernel<T, D>), dim3(a.Hq, a.B), dim3(D), 0, s, a);
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

}  // namespace

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
