// hbm_read_probe.hip -- the measurement aids behind include/gsa_probe.h: a
// streaming-read kernel (the achievable HBM read bandwidth) and a bounded
// spin kernel (keeps the GPU busy while the host queues a timed region).
#include <hip/hip_runtime.h>

#include "gsa_probe.h"

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

// Workgroup g reads the contiguous chunks [g * seg, min((g + 1) * seg, n))
// (16 bytes each), kUnroll coalesced loads per thread per step, with the
// non-temporal hint (a streaming read; measured the fastest form on MI355X).
__global__ __launch_bounds__(kBlock) void read_probe(const u32x4_t* __restrict__ src, int64_t n,
                                                     int64_t seg, uint32_t* sink) {
  const int64_t begin = (int64_t)blockIdx.x * seg;
  const int64_t end = begin + seg < n ? begin + seg : n;
  uint32_t acc = 0;
  int64_t base = begin;
  for (; base + kUnroll * kBlock <= end; base += kUnroll * kBlock) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_nontemporal_load(src + base + u * kBlock + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int64_t i = base + threadIdx.x; i < end; i += kBlock) {
    const u32x4_t v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// One wave spins until `ticks` wall-clock ticks have passed since it started.
// The bound is the argument itself, so the kernel always ends.
__global__ __launch_bounds__(64) void spin_probe(uint64_t ticks) {
  const uint64_t t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(32);
}

}  // namespace

extern "C" int gsa_probe_spin(uint32_t us, void* stream) {
  if (us == 0 || us > 1000000u) return -1;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
      khz <= 0)
    return -3;
  const uint64_t ticks = (uint64_t)us * (uint64_t)khz / 1000u;
  hipLaunchKernelGGL(spin_probe, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), ticks);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int gsa_probe_read(const void* src, size_t bytes, uint32_t* sink, int grid,
                              void* stream) {
  if (!src || !sink || grid < 1 || bytes % 16 != 0 || bytes / 16 >= ((size_t)1 << 31) ||
      ((uintptr_t)src & 15) != 0)
    return -1;
  const int64_t n = (int64_t)(bytes / 16);
  const int64_t seg = (n + grid - 1) / grid;
  hipLaunchKernelGGL(read_probe, dim3((unsigned)grid), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(src), n, seg,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
