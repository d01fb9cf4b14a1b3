// Small gfx950 device helpers shared by the HIP kernels: LDS-direct loads,
// explicit vector-memory waits and a barrier without a memory fence.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mis {

// Fourth descriptor word of a raw (stride 0) buffer resource on CDNA: 32-bit
// data format, so offsets are in bytes and out-of-range reads return zero.
constexpr int kRsrcWord3 = 0x00020000;

// s_waitcnt immediate: at most n vector-memory operations of this wave
// outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int waitcnt_vm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

// LDS-direct buffer load of 16 bytes per lane: lane l's bytes land at lds + 16*l.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, void *lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds, 16, voff,
                                           0, 0, 0);
}

// LDS-direct global load of 16 bytes per lane (per-lane 64-bit address).
__device__ __forceinline__ void lds_load16(const void *src, void *lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// Byte offset of a __shared__ address inside the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)p));
}

// Workgroup barrier without the release/acquire fence of __syncthreads():
// with LDS-direct loads in flight that fence waits for every outstanding
// vector-memory operation. Callers order memory themselves: s_waitcnt for
// their own LDS-direct loads before the barrier, and LDS reads of a buffer
// consumed (by the MFMAs that need them) before the barrier that frees it.
__device__ __forceinline__ void barrier_no_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace mis
