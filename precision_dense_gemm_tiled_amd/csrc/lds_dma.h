// gfx950 helpers shared by the kernels that move global memory straight into
// LDS (global_load_lds) and synchronise on it by hand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mpg {

// One 16-byte direct-to-LDS load: lane l of the wavefront writes its 16 bytes
// at lds + 16 * l (lds must be the same for every lane).
__device__ __forceinline__ void dma16(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// s_waitcnt immediate for "at most VM vector-memory operations outstanding,
// all LDS operations done" (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 left at its maximum, lgkmcnt 11:8). The compiler does not track
// direct-to-LDS loads, so their consumers wait with this explicitly.
template <int VM>
__device__ __forceinline__ void wait_vm_lds() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    constexpr int imm = (VM & 15) | ((VM >> 4) << 14) | (7 << 4);
    __builtin_amdgcn_s_waitcnt(imm);
}

// wait_vm_lds for a count known only after loop unrolling (n folds to a
// constant there, and the recursion to the one matching wait).
template <int N = 63>
__device__ __forceinline__ void wait_vm_lds_n(int n) {
    if constexpr (N >= 0) {
        if (n == N)
            wait_vm_lds<N>();
        else
            wait_vm_lds_n<N - 1>(n);
    }
}

// s_waitcnt for "all LDS operations done", vector-memory loads left in
// flight (vmcnt at its maximum).
__device__ __forceinline__ void wait_lds_only() {
    constexpr int imm = 15 | (3 << 14) | (7 << 4);
    __builtin_amdgcn_s_waitcnt(imm);
}

// Workgroup barrier that publishes LDS-DMA data without waiting for every
// outstanding load: the caller's wait_vm_lds<> decides which loads must have
// landed. Compiler-level fences keep memory operations on their side.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace mpg
