// Building blocks of the LDS pipelines shared by the router and the grouped
// GEMMs: asynchronous global -> LDS copies, counted waits, fence-free
// workgroup barriers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lbv {

// Waits until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Waits until every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

// Workgroup barrier without the memory fence that __syncthreads() implies (the
// fence would wait for every load in flight, i.e. drain the prefetch queue).
// The empty asm keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Asynchronous 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4):
// lane l's 16 bytes land at LDS byte address lds_base + 16 l.  Written as asm
// so that the compiler's wait-count pass, which cannot tell the stage being
// filled from the stage being read, does not drain the queue before every LDS
// read; the kernel orders these copies itself (wait_vmcnt + block_barrier).
// The instruction has no register results.
__device__ __forceinline__ void lds_dma16(const void* gsrc, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(lds_base), "v"(gsrc)
        : "memory", "m0");
}

// Same copy with the source given as a wave-uniform 64-bit base (scalar
// registers) plus a 32-bit per-lane byte offset, and the LDS destination as a
// wave-uniform base plus a compile-time byte offset.
template <uint32_t LDS_OFF>
__device__ __forceinline__ void lds_dma16_sb(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile(
        "s_add_u32 m0, %0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(lds_base), "v"(voff), "s"(sbase), "i"(LDS_OFF)
        : "memory", "m0", "scc");
}

// 4-byte-per-lane variant (global_load_lds_dword): lane l's word lands at
// LDS byte address lds_base + 4 l.
__device__ __forceinline__ void lds_dma4_sb(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, %2"
        :
        : "s"(lds_base), "v"(voff), "s"(sbase)
        : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

}  // namespace lbv
