// LDS staging and wait helpers shared by the matrix-core kernels of libtp
// (gfx950): buffer resources, the buffer-load-to-LDS path, vector-memory
// counter waits and an LDS-only workgroup barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

#define TP_LDS __attribute__((address_space(3)))

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS only (global loads stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw buffer resource over [base, base + bytes): loads past the end read as
// zero (and write zeros into LDS on the load-to-LDS path).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: raw (untyped) 32-bit data format on gfx9-family parts
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// One wave instruction moves 64 x 16 bytes from global memory into LDS: lane i
// reads 16 bytes at voff + soff of the resource and lands at lds + 16*i.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (TP_LDS void*)lds, 16, (int)voff, (int)soff, 0, 0);
}

constexpr uint32_t kOob = 0x80000000u;  // beyond every range: reads as zero

}  // namespace tp
