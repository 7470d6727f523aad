// lds_dma.hpp — direct global -> LDS copies (gfx950 global_load_lds), the waits
// and barriers that order them, and LDS reads of what they filled.
#pragma once

#include "device.hpp"

namespace pf {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

__device__ __forceinline__ void dma16(const int8_t* g, int8_t* lds_base)
{
    __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_base, 16, 0, 0);
}

__device__ __forceinline__ void dma4(const float* g, int8_t* lds_base)
{
    __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_base, 4, 0, 0);
}

// s_waitcnt with only the vector-memory counter limited to N (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt with only the LDS counter limited to 0 (vmcnt and expcnt at their
// maxima): this wave's LDS reads and writes have completed.
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
}

// Workgroup barrier without the memory fence of __syncthreads (which would wait
// for every outstanding load, draining the DMA pipeline).  Completion of this
// wave's DMAs is established by wait_vmcnt before it; the signal fences keep
// the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void stage_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// LDS reads of DMA-filled buffers.  The compiler's wait-count pass cannot tell
// which LDS bytes an LDS DMA writes, so in front of an LDS read that it can see
// it may wait for every DMA still in flight (vmcnt(0)), which empties the ring
// each stage.  These reads are inline assembly, invisible to that pass, and end
// with their own lgkmcnt(0); that the DMA data has landed is the caller's
// vmcnt wait (its own wave's DMAs) or a barrier after one (other waves').
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ v4f lds_read_v4f(uint32_t a)
{
    v4f r;
    asm volatile("ds_read_b128 %0, %1\n"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r) : "v"(a));
    return r;
}

__device__ __forceinline__ float lds_read_f32(uint32_t a)
{
    float r;
    asm volatile("ds_read_b32 %0, %1\n"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r) : "v"(a));
    return r;
}

}  // namespace pf
