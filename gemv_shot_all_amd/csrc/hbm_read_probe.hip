// hbm_read_probe.hip -- the streaming-read kernel behind include/gsa_probe.h
// (a measurement aid for the achievable HBM read bandwidth).
#include <hip/hip_runtime.h>

#include "gsa_probe.h"

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_probe(const uint4* __restrict__ src, int64_t n,
                                                  uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int gsa_probe_read(const void* src, size_t bytes, uint32_t* sink, int grid,
                              void* stream) {
  if (!src || !sink || grid < 1 || bytes % 16 != 0 || bytes / 16 >= ((size_t)1 << 31) ||
      ((uintptr_t)src & 15) != 0)
    return -1;
  hipLaunchKernelGGL(read_probe, dim3((unsigned)grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                     (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
