// mfma_rate.hip - matrix-core probe: how fast this device sustains bf16 MFMA work and at
// what shader clock.  It is the measured reference next to the nominal 2.5 PFLOP/s
// (which assumes 2.4 GHz) against which the prefill's and the verifier's TFLOP/s are
// read; it is not part of the method.
//
// Every wave runs `iters` rounds of four independent v_mfma_f32_32x32x16_bf16 on
// register operands, so the matrix core never waits on a dependency or on memory, then
// writes one float per lane so the work is kept.  The first wave of work-group 0 also
// records the shader-clock (s_memtime) and 100 MHz real-time (s_memrealtime) ticks its
// loop took: their ratio is the shader clock under this load.
#include "masw_internal.hpp"

namespace masw {
namespace {

constexpr int kRateThreads = 256;

typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef float rf32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kRateThreads) void mfma_rate_kernel(float* out, int iters, uint64_t* clocks) {
  const int lane = threadIdx.x & 63;
  rbf16x8_t x, y;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = __bf16(0.0078125f * float((lane + i) & 7));
    y[i] = __bf16(0.0078125f * float((lane * 3 + i) & 7));
  }
  rf32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c3, 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += (c0[i] + c1[i]) + (c2[i] + c3[i]);
  out[size_t(blockIdx.x) * kRateThreads + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = t1 - t0;
    clocks[1] = r1 - r0;
  }
}

}  // namespace

int launch_mfma_rate(int work_groups, int iters, float* out, uint64_t* clocks, hipStream_t s) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(work_groups), dim3(kRateThreads), 0, s, out, iters, clocks);
  return hipGetLastError() == hipSuccess ? MASW_OK : MASW_ERR_LAUNCH;
}

}  // namespace masw
