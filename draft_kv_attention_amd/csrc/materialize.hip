// materialize.hip - mirrored slot projection (Technical Review §3.2, Algorithm 1
// step 3): K_g = H W_K,g and V_g = H W_V,g, written into slot row m-1 of every KV head
// (head k = columns k*D .. k*D+D-1), plus the per-sequence boundary decision that
// gates the slot query launched after it.
//
// bf16: a dense contraction on the matrix cores.  Each work-group owns 64 output
// columns of one matrix and all hidden rows; its 16 waves split the hidden dimension.
// Per 32-row step a wave loads a [32 k][64 n] weight tile with fully coalesced 16-byte
// loads, writes it transposed into its own LDS tile, and feeds four
// v_mfma_f32_16x16x32_bf16 (A = H rows, zero-padded to 16; B = the transposed tile).
// The 16 wave partials are summed in LDS in a fixed order (deterministic).
// fp32 caches (small models) use a plain per-column VALU loop.
#include "masw_internal.hpp"

namespace masw {
namespace {

// Slot index m this call materializes for sequence b, or 0.  Only a boundary step
// t = S + W + m r with n_slots == m - 1 acts; n_slots == m means already done.
__device__ __forceinline__ int boundary_slot(const ProjectArgs& a, int b, int& bits) {
  const int t = a.seq_len[b];
  const int d = t - a.g.S - a.g.W;
  if (d < a.g.r || d % a.g.r) return 0;
  const int m = d / a.g.r;
  const int have = a.n_slots[b];
  if (have == m) return 0;
  if (have != m - 1) { bits |= MASW_DEV_SLOT_MISSING; return 0; }
  if (m > a.g.max_slots) { bits |= MASW_DEV_SLOT_CAPACITY; return 0; }
  return m;
}

constexpr int kCols = 64;        // output columns per work-group
constexpr int kWaves = 16;
constexpr int kStepK = 32;       // hidden rows per MFMA step
constexpr int kTRow = kStepK + 8;  // transposed tile row (bf16), padded: 80 bytes

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t u16_of(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

__global__ __launch_bounds__(kWaves * kWave) void project_mfma_kernel(const ProjectArgs a) {
  const int nblk = blockIdx.x, which = blockIdx.y, z = blockIdx.z;
  const int N = a.Hkv * a.D;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

  __shared__ int sm_m[16];
  __shared__ int sm_any;
  __shared__ __attribute__((aligned(16))) uint16_t smem[kWaves * kCols * kTRow];

  if (tid == 0) sm_any = 0;
  __syncthreads();
  if (tid < 16) {
    const int b = z * 16 + tid;
    int bits = 0, m = 0;
    if (b < a.B) m = boundary_slot(a, b, bits);
    sm_m[tid] = m;
    if (m) atomicOr(&sm_any, 1);
    if (nblk == 0 && which == 0 && b < a.B) {
      a.active[b] = m;
      if (bits) atomicOr(a.err, bits);
    }
  }
  __syncthreads();
  if (!sm_any) return;

  const uint16_t* Wm = static_cast<const uint16_t*>(which ? a.w_v : a.w_k);
  const uint16_t* H = static_cast<const uint16_t*>(a.h);
  uint16_t* wt = smem + wave * kCols * kTRow;
  const int iters = (a.hidden + kWaves * kStepK - 1) / (kWaves * kStepK);
  const int brow = z * 16 + (lane & 15);
  const int col8 = lane & 7, kq = lane >> 3;   // loader: 8 lanes per 128-byte row segment

  f32x4_t acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < iters; ++it) {
    const int kk = (wave * iters + it) * kStepK;
    uint4 wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = kk + 4 * kq + i;
      wv[i] = k < a.hidden
                  ? *reinterpret_cast<const uint4*>(Wm + size_t(k) * N + nblk * kCols + col8 * 8)
                  : make_uint4(0, 0, 0, 0);
    }
    // transposed store: tile row n holds 32 consecutive k of column n
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint2 x;
      x.x = u16_of(wv[0], e) | (u16_of(wv[1], e) << 16);
      x.y = u16_of(wv[2], e) | (u16_of(wv[3], e) << 16);
      *reinterpret_cast<uint2*>(wt + (col8 * 8 + e) * kTRow + 4 * kq) = x;
    }
    uint4 av = make_uint4(0, 0, 0, 0);
    const int ka = kk + (lane >> 4) * 8;
    if (brow < a.B && ka < a.hidden) av = *reinterpret_cast<const uint4*>(H + size_t(brow) * a.hidden + ka);
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const uint4 bv = *reinterpret_cast<const uint4*>(wt + (nt * 16 + (lane & 15)) * kTRow + (lane >> 4) * 8);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                        __builtin_bit_cast(bf16x8_t, bv), acc[nt], 0, 0, 0);
    }
    __syncthreads();
  }

  // D layout of a 16x16 MFMA: lane holds rows 4*(lane/16)+i of column lane%16.
  float* red = reinterpret_cast<float*>(smem);   // [waves][16 rows][64 cols]
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      red[(wave * 16 + (lane >> 4) * 4 + i) * kCols + nt * 16 + (lane & 15)] = acc[nt][i];
  __syncthreads();
  const int row = tid / kCols, col = tid % kCols;
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += red[(w * 16 + row) * kCols + col];
  const int b = z * 16 + row;
  const int m = sm_m[row];
  if (b < a.B && m > 0) {
    const int n = nblk * kCols + col;
    const int kvh = n / a.D, d = n - (n / a.D) * a.D;
    uint16_t* dst = static_cast<uint16_t*>(which ? a.v_slot : a.k_slot);
    dst[((size_t(b) * a.Hkv + kvh) * a.g.max_slots + (m - 1)) * a.D + d] = f32_to_bf16(s);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void project_valu_kernel(const ProjectArgs a) {
  const int b = blockIdx.y;
  const int N = a.Hkv * a.D;
  int bits = 0;
  const int m = boundary_slot(a, b, bits);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.active[b] = m;
    if (bits) atomicOr(a.err, bits);
  }
  if (!m) return;
  const int col = blockIdx.x * blockDim.x + threadIdx.x;
  if (col >= 2 * N) return;
  const int which = col / N, n = col - which * N;
  const T* Wm = static_cast<const T*>(which ? a.w_v : a.w_k);
  const T* H = static_cast<const T*>(a.h) + size_t(b) * a.hidden;
  float s = 0.f;
  for (int k = 0; k < a.hidden; ++k) s = fmaf(Elem<T>::to_f32(H[k]), Elem<T>::to_f32(Wm[size_t(k) * N + n]), s);
  const int kvh = n / a.D, d = n - kvh * a.D;
  T* dst = static_cast<T*>(which ? a.v_slot : a.k_slot);
  dst[((size_t(b) * a.Hkv + kvh) * a.g.max_slots + (m - 1)) * a.D + d] = Elem<T>::from_f32(s);
}

}  // namespace

int launch_project(const ProjectArgs& a, int dtype, hipStream_t s) {
  const int N = a.Hkv * a.D;
  if (dtype == MASW_BF16) {
    hipLaunchKernelGGL(project_mfma_kernel, dim3(N / kCols, 2, (a.B + 15) / 16), dim3(kWaves * kWave), 0, s, a);
  } else {
    hipLaunchKernelGGL(project_valu_kernel<float>, dim3((2 * N + 255) / 256, a.B), dim3(256), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? MASW_OK : MASW_ERR_LAUNCH;
}

}  // namespace masw
