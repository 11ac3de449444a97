// Direct global-to-LDS loads (gfx950 global_load_lds_dwordx4 and
// buffer_load_dwordx4 ... lds).
#pragma once

#include <hip/hip_runtime.h>

namespace qtalk {

// one 16-byte direct-to-LDS load per lane: lane l's bytes land at lds + 16 l
// (lds uniform across the wave).  The load counts on vmcnt like any vector
// load; the LDS data is there once it retires.  A helper function, not a
// lambda: a lambda holding this builtin makes the host pass drop the
// kernel's launch stub.
__device__ __forceinline__ void lds_load16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// Buffer resource over `bytes` bytes from `base`: raw addressing (stride 0),
// word 3 = 0x00020000 (the gfx9 raw-buffer format: 32-bit data, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// The same 16-byte load through a buffer resource: lane l reads bytes
// [voff + soff, +16) of the resource (voff per lane, soff wave-uniform and
// held in a scalar register), so a loop that walks a buffer advances soff
// and spends no vector instruction on addresses.  Bytes past the resource's
// size read as zero.
__device__ __forceinline__ void lds_load16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

}  // namespace qtalk
