// memops.h -- buffer resources, explicit vector-memory waits and a bare
// workgroup barrier, shared by the kernels that keep loads in flight across
// a barrier.
#pragma once

#include "common.h"

namespace moeq {

typedef __attribute__((address_space(3))) void lds_void_t;

// A buffer resource over [base, base + bytes).  The hardware checks the range
// per dword, so the range is rounded up to the 16-byte granule holding the
// last byte (arrays start 16-byte aligned, so the extra bytes never leave
// that granule, nor its page).  A read past the range returns zeros.
__device__ inline __amdgpu_buffer_rsrc_t rsrc_of(const void *base, uint64_t bytes) {
    bytes = (bytes + 15u) & ~(uint64_t)15u;
    const u32 n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (u32)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, 0x00020000);
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
// Emitted through the builtin so that the compiler's own wait insertion knows
// which loads are complete (an s_waitcnt in inline assembly is opaque to it);
// the clobber keeps memory accesses on their side.  Encoding (gfx9): vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima.
template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// Workgroup barrier that leaves vector loads in flight.  __syncthreads()
// carries release/acquire fences that make the compiler wait for every
// outstanding vector load (vmcnt(0)); this one only completes the wave's LDS
// operations before the barrier.  The memory clobbers keep LDS accesses on
// their side of it.
__device__ inline void ring_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace moeq
