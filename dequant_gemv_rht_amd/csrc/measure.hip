// The streaming-read ceiling (include/wq_measure.h): one 256-thread
// workgroup per 8 KiB, two 16-byte loads per lane, no stores but a guard
// that keeps the loads.
#include "wq_internal.h"

namespace wq {
namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ p, size_t n16,
                                                          uint32_t *sink) {
  const size_t i0 = (size_t)blockIdx.x * 512 + threadIdx.x;
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const size_t i = i0 + (size_t)u * 256;
    if (i < n16) {
      const uint4 v = p[i];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t s) {
  const size_t n16 = bytes / 16, blocks = (n16 + 511) / 512;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint4 *>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace wq

