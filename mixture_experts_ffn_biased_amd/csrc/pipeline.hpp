// Helpers for gfx950 kernels that stage tiles through LDS with direct
// global-to-LDS loads (global_load_lds_dwordx4, or buffer_load_dwordx4 ...
// lds through a buffer resource) in a ring of separate __shared__ slots.  The wait counts are explicit: a stage is complete once
// at most the loads issued after it are outstanding (loads complete in
// order), and the barrier is a bare s_barrier, which does not wait for the
// in-flight LDS loads the way __syncthreads() does.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((address_space(3))) void lds_void;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that neither waits for the in-flight LDS loads nor lets
// the compiler move memory accesses across it.
__device__ __forceinline__ void raw_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Cache-policy operand of a load: the non-temporal hint (gfx950's nt bit),
// for operand streams that should not displace data read again later (the
// weight streams of the decode kernels and of the prefill gate/up kernel).
constexpr int kLoadDefault = 0, kLoadNonTemporal = 2;

// 16 bytes per lane from global memory into LDS at lds + lane * 16.
template <int POLICY = kLoadDefault>
__device__ __forceinline__ void dma16(const void *src, void *lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void *)lds, 16, 0, POLICY);
}

// Raw buffer resource over bytes [base, base + bytes) (bytes < 2^32):
// offsets past the end read zeros instead of faulting.  Word 3 selects
// 32-bit data, the usual setting for raw dword loads on gfx9 parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// The same 16-byte load into LDS through a buffer resource: the base and the
// scalar offset stay in SGPRs, only the 32-bit lane offset is a VGPR.
template <int POLICY = kLoadDefault>
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, void *lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, static_cast<int>(voff), soff, 0, POLICY);
}

}  // namespace moe
