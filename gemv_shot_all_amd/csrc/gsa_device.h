// gsa_device.h -- device helpers shared by the kernels of libgsa (gfx950).
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gsa {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at `base` (raw, stride 0).  A load whose
// per-lane offset is past the end returns zeros instead of touching memory.
// The range check does not cover the uniform (SGPR) offset, so every offset
// below goes into the per-lane one.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes at byte offset off (per lane, range-checked).  Cache policy 2 is
// the non-temporal hint (nt): the weights are streamed once per call, and a
// plain streaming read reaches markedly more HBM bandwidth with it on MI355X.
#ifndef GSA_A_CPOL
#define GSA_A_CPOL 2
#endif
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, GSA_A_CPOL);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// The same without the hint, for activations (read by every workgroup: kept
// cached).
__device__ __forceinline__ uint4 buf_load16_cached(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Agent-scope (device-coherent) relaxed accesses for protocol state.
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_flag(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until at most N vector memory operations of this wave are still
// outstanding (s_waitcnt vmcnt(N), expcnt and lgkmcnt untouched; gfx9
// encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_vm_all() { wait_vm_le<0>(); }

// Copy 16 bytes per active lane from global memory straight into LDS: lane l
// writes lds_base + 16 * l (lds_base is wave-uniform).  Completion is counted
// by vmcnt like any other vector load.  CPOL: cache policy (2: the
// non-temporal hint, for data streamed once).
template <int CPOL = 0>
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(
      (const void __attribute__((address_space(1)))*)src,
      (void __attribute__((address_space(3)))*)lds_base, 16, 0, CPOL);
}

}  // namespace
}  // namespace gsa
