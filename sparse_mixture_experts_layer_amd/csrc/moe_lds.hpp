// Primitives of the LDS-staged MFMA kernels: wave-wide global->LDS fragment
// loads, a barrier that leaves in-flight loads alone, and explicit waits.
#pragma once

#include "moe_common.hpp"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// One wave-wide 16-byte-per-lane load of (src + OFF) into LDS at lds + OFF
// (+ 16 * lane); OFF is an immediate, applied by the instruction to both
// addresses.
template <int OFF>
__device__ __forceinline__ void load_frag(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)lds, 16, OFF, 0);
}

// Workgroup barrier without a memory fence: __syncthreads' release fence
// would drain every outstanding global->LDS load, including the stages
// prefetched for later steps.  The compiler-only fences keep LDS accesses on
// their side; the builtin (unlike an inline-asm s_barrier, which the compiler
// must treat as reading every accumulator) does not drain in-flight MFMAs.
__device__ __forceinline__ void barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt vmcnt(n) lgkmcnt(0) through the builtin, so the compiler sees it
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
__device__ __forceinline__ void wait_vm_lgkm0(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0070); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0072); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0074); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0075); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0076); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0078); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x007A); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x007C); break;
    case 16: __builtin_amdgcn_s_waitcnt(0x4070); break;
    case 18: __builtin_amdgcn_s_waitcnt(0x4072); break;
    default: __builtin_amdgcn_s_waitcnt(0x0070); break;  // stricter than asked: always safe
  }
}

}  // namespace moe
