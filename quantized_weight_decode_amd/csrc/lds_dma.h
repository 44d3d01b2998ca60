// lds_dma.h -- loads from global memory straight into LDS on gfx950, with the
// waits placed by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qh {

// Byte offset of an LDS object within the workgroup's LDS allocation: the
// value M0 takes for a load straight into LDS.
__device__ __forceinline__ uint32_t lds_byte_offset(const void* p) {
    typedef __attribute__((address_space(3))) const void* lds_cptr;
    return (uint32_t)(uintptr_t)(lds_cptr)p;
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l's bytes at base + voff land at LDS byte
// m0 + 16 l, with base and m0 wave-uniform (SGPRs) and voff the lane's
// 32-bit byte offset. The load is written as inline asm so that the compiler
// does not track it: once it sees such a load in flight, it waits for every
// outstanding vector-memory instruction before any LDS read, which leaves no
// load in flight across a computation. The caller therefore orders the bytes
// itself: wait_vmcnt<N>() before the first LDS read of them (by this wave;
// other waves read them after a barrier that follows that wait), N counting
// every vector-memory load issued after this one. Loads, these included,
// complete in order among themselves, so with at most N left this one has
// landed; stores, which may complete out of order with loads, can only make
// the wait longer. The compiler's own waits stay correct for the same
// reason (the loads it does not see only make them longer), but a wait it
// places after such a load also waits for it: issue these after the first
// use of any register load still in flight, which `after`, a value computed
// from that use, enforces (an asm input the instruction does not read). M0
// is restored; the one wait state between writing M0 and the load reading
// it is the s_nop.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t m0,
                                          uint32_t after = 0u) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(base), "s"(m0), "v"(after)
        : "memory");
}

// s_waitcnt vmcnt(N): at most N vector-memory instructions of this wave left
// in flight. A compiler barrier for memory accesses as well.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit count");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace qh
