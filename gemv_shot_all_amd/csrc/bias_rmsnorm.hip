// bias_rmsnorm.hip -- the fused epilogue's bias + RMSNorm as a kernel of its
// own (gfx950): the unfused form, a plain GEMV + all-reduce call followed by
// this kernel on the same stream ("PyTorch Symmetric Memory: A New
// Programming Paradigm for Distributed AI" talk, real-model example: the
// reduction, a bias addition and an RMSNorm, there fused into one kernel).
// Same definition as the fused call (RMSNorm over the N rows of each token
// column; fp32 throughout):
//   z[n][b] = out[n][b] + bias[n];  inv[b] = 1 / sqrtf(sum_n z^2 / N + eps);
//   y[n][b] = (z[n][b] * inv[b]) * w[n]  (fp32, or rounded to bf16).
// One workgroup per column b: thread t takes rows t, t + T, ... in ascending
// order (eight loads in flight before their additions), the lanes of a wave
// are summed by a fixed butterfly and the waves in wave order, so inv is the
// same bits on every call; y is then computed from it exactly as the fused
// call computes it from its own inv.

#include "gsa_device.h"
#include "gsa_internal.h"

namespace gsa {
namespace {

constexpr int kRmsThreads = 1024;
constexpr int kRmsBatch = 8;  // rows per thread with their loads in flight together

__device__ __forceinline__ uint16_t rms_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__global__ __launch_bounds__(kRmsThreads) void bias_rmsnorm_kernel(
    const float* out, int64_t N, int B, const float* bias, const float* w, float eps, void* y,
    int y_bf16, float* inv_rms) {
  __shared__ float wsum[kRmsThreads / 64];
  __shared__ float s_inv;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int64_t kStep = (int64_t)kRmsThreads * kRmsBatch;

  float acc = 0.0f;
  for (int64_t n0 = tid; n0 < N; n0 += kStep) {
    float z[kRmsBatch];
#pragma unroll
    for (int u = 0; u < kRmsBatch; ++u) {
      const int64_t n = min(n0 + (int64_t)u * kRmsThreads, N - 1);
      z[u] = out[n * B + b] + (bias ? bias[n] : 0.0f);
    }
#pragma unroll
    for (int u = 0; u < kRmsBatch; ++u)
      if (n0 + (int64_t)u * kRmsThreads < N) acc = acc + z[u] * z[u];
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) acc = acc + __shfl_xor(acc, m);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.0f;
    for (int v = 0; v < kRmsThreads / 64; ++v) tot = tot + wsum[v];
    const float inv = 1.0f / sqrtf(tot / (float)N + eps);
    s_inv = inv;
    if (inv_rms) inv_rms[b] = inv;
  }
  __syncthreads();
  const float inv = s_inv;

  for (int64_t n0 = tid; n0 < N; n0 += kStep) {
    float z[kRmsBatch], wv[kRmsBatch];
#pragma unroll
    for (int u = 0; u < kRmsBatch; ++u) {
      const int64_t n = min(n0 + (int64_t)u * kRmsThreads, N - 1);
      z[u] = out[n * B + b] + (bias ? bias[n] : 0.0f);
      wv[u] = w ? w[n] : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < kRmsBatch; ++u) {
      const int64_t n = n0 + (int64_t)u * kRmsThreads;
      if (n < N) {
        float v = z[u] * inv;
        if (w) v = v * wv[u];
        if (y_bf16)
          static_cast<uint16_t*>(y)[n * B + b] = rms_bf16_rne(v);
        else
          static_cast<float*>(y)[n * B + b] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_bias_rmsnorm(const float* out, int64_t N, int B, const float* bias,
                               const float* w, float eps, void* y, bool y_bf16, float* inv_rms,
                               hipStream_t s) {
  hipLaunchKernelGGL(bias_rmsnorm_kernel, dim3((unsigned)B), dim3(kRmsThreads), 0, s, out, N, B,
                     bias, w, eps, y, y_bf16 ? 1 : 0, inv_rms);
  return hipGetLastError();
}

}  // namespace gsa
