// lds_dma.h -- gfx950 direct global->LDS loads and the wave-uniform values
// they need, shared by the grouped-GEMM and router-GEMM kernels.
#pragma once
#include "moe_internal.h"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Values every lane of a wave holds equally, made visible to the compiler as
// such (scalar registers): buffer descriptors and the LDS target of a direct
// load must be wave-uniform, otherwise the compiler wraps the load in a
// per-lane loop.
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t wave_uniform(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}
template <typename T>
__device__ __forceinline__ T* wave_uniform(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = wave_uniform(static_cast<uint32_t>(v));
  const uint32_t hi = wave_uniform(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Raw buffer resource over [base, base + bytes) (gfx9 descriptor: no
// swizzle, 32-bit data); loads past `bytes` return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(wave_uniform(base)), 0,
                                           wave_uniform(bytes), 0x00020000);
}

// One wave moves 1 KiB straight into LDS: lane i's 16 bytes, read at
// voffset (per lane) + soffset (wave-uniform) inside the buffer, land at
// lds_group + 16 * i.  Callers pick voffset so that the XOR swizzle of their
// LDS layout holds the right chunk at each physical position.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t soffset,
                                      bf16_t* lds_group) {
  // lds_group is derived from the wave index made uniform by the caller
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_group, 16, voffset,
                                           wave_uniform(soffset), 0, 0);
}

// s_waitcnt lgkmcnt(0): every LDS read this wave issued has returned (vmcnt
// and expcnt unconstrained; gfx9 encoding)
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// s_waitcnt with vmcnt <= n, expcnt and lgkmcnt unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace moe
