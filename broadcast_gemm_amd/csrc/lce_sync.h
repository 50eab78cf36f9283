// lce_sync.h -- wave-level synchronisation helpers shared by the persistent LCE engines that
// stream activations with direct-to-LDS loads: flag loads and stores for the user/candidate
// hand-off, the bare workgroup barrier, and vector-memory waits the compiler can see.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ikbo {

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t ld_flag(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup barrier without the fences of __syncthreads, which would also wait for every
// load the wave has in flight (the ring's opening steps).  Callers wait for the LDS writes
// they publish (direct-to-LDS loads: vmcnt) before it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt through the builtin rather than inline asm, so that the compiler's own wait
// insertion sees it: the compiler guards every LDS read with a wait for the direct-to-LDS loads
// it cannot rule out, and a wait it cannot see leaves that guard at vmcnt(0), which would also
// wait for the HBM reads of the ring.  The empty asm keeps memory operations on their side.
// Field layout: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }
template <int K>
__device__ __forceinline__ void vm_wait() {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(K, 15));
    asm volatile("" ::: "memory");
}

// vmcnt(n) for a run-time n: the counter field is an immediate, so this switches over the
// values the counter can hold (it saturates at 63: a wave never has more memory operations
// outstanding, so waiting for 63 waits for nothing).
__device__ __forceinline__ void vm_wait_dyn(int n) {
    n = (int)__builtin_amdgcn_readfirstlane(n);
    switch (n < 63 ? n : 63) {
#define IKBO_VMW(k) case k: vm_wait<k>(); break;
#define IKBO_VMW8(k) IKBO_VMW(k) IKBO_VMW(k + 1) IKBO_VMW(k + 2) IKBO_VMW(k + 3) IKBO_VMW(k + 4) IKBO_VMW(k + 5) \
    IKBO_VMW(k + 6) IKBO_VMW(k + 7)
        IKBO_VMW8(0) IKBO_VMW8(8) IKBO_VMW8(16) IKBO_VMW8(24) IKBO_VMW8(32) IKBO_VMW8(40) IKBO_VMW8(48)
        IKBO_VMW(56) IKBO_VMW(57) IKBO_VMW(58) IKBO_VMW(59) IKBO_VMW(60) IKBO_VMW(61) IKBO_VMW(62)
#undef IKBO_VMW8
#undef IKBO_VMW
        default: break;
    }
}

}  // namespace ikbo
