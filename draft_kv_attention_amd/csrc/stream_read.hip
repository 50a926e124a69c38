// stream_read.hip - streaming-read probe: how fast a plain kernel reads HBM on this
// device.  It is the measured reference next to the nominal 8 TB/s against which the
// attention kernels' achieved GB/s are read; it is not part of the method.
//
// Each work-group reads one contiguous chunk of 16-byte words with kUnroll loads in
// flight per lane (non-temporal, like the attention kernels' K/V streams), adds the 32-bit words modulo 2^32, reduces across the work-group
// through LDS and adds its total into sums[blockIdx % MASW_STREAM_SUMS] with one atomic
// (spread so that the atomics of thousands of work-groups do not queue on one word).
#include "masw_internal.hpp"

namespace masw {
namespace {

constexpr int kReadThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4_t* __restrict__ p, long n16,
                                                                   long per_wg, uint32_t* sum) {
  const long base = long(blockIdx.x) * per_wg;
  const long end = min(base + per_wg, n16);
  uint32_t acc = 0;
  for (long i = base + threadIdx.x; i < end; i += long(kReadThreads) * kUnroll) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long j = i + long(kReadThreads) * u;
      v[u] = j < end ? __builtin_nontemporal_load(&p[j]) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc += v[u].x + v[u].y + v[u].z + v[u].w;
  }
  __shared__ uint32_t part[kReadThreads / kWave];
  for (int o = kWave / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kReadThreads / kWave; ++w) t += part[w];
    atomicAdd(&sum[blockIdx.x % MASW_STREAM_SUMS], t);
  }
}

}  // namespace
}  // namespace masw

extern "C" MASW_API int masw_stream_read(const void* p, size_t bytes, int32_t work_groups, uint32_t* sums,
                                         hipStream_t stream) {
  if (!p || !sums || bytes == 0 || bytes % 16 != 0 || work_groups < 0) return MASW_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(p) & 15) != 0) return MASW_ERR_ARG;
  const long n16 = long(bytes / 16);
  const long wgs = work_groups > 0 ? work_groups : 2048;
  const long per = (n16 + wgs - 1) / wgs;
  hipLaunchKernelGGL(masw::stream_read_kernel, dim3(unsigned(wgs)), dim3(masw::kReadThreads), 0, stream,
                     static_cast<const masw::u32x4_t*>(p), n16, per, sums);
  return hipGetLastError() == hipSuccess ? MASW_OK : MASW_ERR_LAUNCH;
}
