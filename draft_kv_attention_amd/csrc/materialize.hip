// materialize.hip - mirrored slot projection (Technical Review §3.2, Algorithm 1
// step 3): K_g = H W_K,g and V_g = H W_V,g, written into slot row m-1 of every KV head
// (head k = columns k*D .. k*D+D-1), plus the per-sequence boundary decision that
// gates the slot query launched after it.
//
// bf16: a dense contraction on the matrix cores, spread over 64-column blocks, the two
// matrices and up to kMaxProjectSplits slices of the hidden dimension (256 work-groups
// at the 3B shape); see project_mfma_kernel.
// fp32 caches (small models) use a plain per-column VALU loop.
#include "project_mfma.hpp"

namespace masw {
namespace {

using namespace proj;

template <int RG>
__global__ __launch_bounds__(kPWaves * kWave) void project_mfma_kernel(const ProjectArgs a) {
  __shared__ ProjectLds<RG> lds;
  project_mfma_body<RG>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds);
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
  const bool live = col < 2 * N;
  const int which = col / N, n = col - which * N;
  float s = 0.f;
  if (live) {
    const T* Wm = static_cast<const T*>(which ? a.w_v : a.w_k);
    const T* H = static_cast<const T*>(a.h) + size_t(b) * a.hidden;
    for (int k = 0; k < a.hidden; ++k) s = fmaf(Elem<T>::to_f32(H[k]), Elem<T>::to_f32(Wm[size_t(k) * N + n]), s);
  }
  const int kvh = n / a.D, d = n - kvh * a.D;
  if (a.rope_theta > 0.f) {
    // a block is 256 columns starting at a multiple of 256 and D divides 256, so the
    // partner column (d ^ D/2, or d ^ 1) is in the block
    __shared__ float xs[256];
    xs[threadIdx.x] = s;
    __syncthreads();
    const float xp = xs[threadIdx.x ^ rope_partner_xor(a.rope_style, a.D)];
    if (live && which == 0)
      s = rope_turn(s, xp, rope_first(d, a.rope_style, a.D), rope_inv_freq(rope_freq(d, a.rope_style, a.D), a.D, a.rope_theta),
                    a.g.S + m * a.g.r);
  }
  if (!live) return;
  T* dst = static_cast<T*>(which ? a.v_slot : a.k_slot);
  dst[((size_t(b) * a.Hkv + kvh) * a.g.max_slots + (m - 1)) * a.D + d] = Elem<T>::from_f32(s);
}

}  // namespace

int launch_project(const ProjectArgs& a, int dtype, hipStream_t s) {
  const int N = a.Hkv * a.D;
  if (dtype == MASW_BF16) {
    if (a.ksplits < 1 || a.ksplits > kMaxProjectSplits || a.k_per_split % (kPWaves * kStepK)) return MASW_ERR_ARG;
    if (a.prefill_ns > 0) {
      if (a.ksplits != 1) return MASW_ERR_ARG;
      const long rows = long(a.B) * a.prefill_ns, per = 16 * kPrefillRowGroups;
      hipLaunchKernelGGL(project_mfma_kernel<kPrefillRowGroups>, dim3(N / kCols, 2, (rows + per - 1) / per),
                         dim3(kPWaves * kWave), 0, s, a);
    } else {
      hipLaunchKernelGGL(project_mfma_kernel<1>, dim3(N / kCols, 2, a.ksplits * ((a.B + 15) / 16)), dim3(kPWaves * kWave), 0,
                         s, a);
    }
  } else {
    if (a.prefill_ns > 0) return MASW_ERR_UNIMPLEMENTED;
    hipLaunchKernelGGL(project_valu_kernel<float>, dim3((2 * N + 255) / 256, a.B), dim3(256), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? MASW_OK : MASW_ERR_LAUNCH;
}

}  // namespace masw
