// Direct global-to-LDS loads (gfx950 global_load_lds_dwordx4).
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

}  // namespace qtalk
