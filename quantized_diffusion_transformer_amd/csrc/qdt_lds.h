// Register-vector types and the inline-asm memory helpers shared by the GEMM kernels: LDS-DMA
// (global memory straight into LDS), explicit load-counter waits, the MFMA drain before
// accumulators are read, and uniform-pointer / LDS-address helpers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qdt {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
// 16-byte chunk as a native vector (HIP's uint4 is a struct whose copies become memcpy,
// which keeps arrays of it out of registers)
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Wait for the MFMA pipeline to drain before accumulators are read by other instructions.
__device__ __forceinline__ void mfma_drain() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Pins a register value after the preceding volatile asm statements (an mfma_drain): the empty asm
// "writes" it, so no read of it can be scheduled above the drain.  Volatile asm statements keep
// their order, so the drain's wait states always separate the last MFMA from the first read.
template <typename T>
__device__ __forceinline__ void keep_after_a(T& v) {
    asm volatile("" : "+a"(v));
}
template <typename T>
__device__ __forceinline__ void keep_after_v(T& v) {
    asm volatile("" : "+v"(v));
}

// LDS-DMA of one dword per lane (global_load_lds_dword): lane l writes LDS m0 + 4 l.
__device__ __forceinline__ void lds_dma4(uint32_t lds_addr, const void* gptr) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_addr), "v"(gptr)
                 : "memory", "m0");
}
// LDS-DMA (gfx950 global_load_lds_dwordx4): lane l of the wave copies 16 bytes from its global
// address to LDS at m0 + 16 l, i.e. one wave instruction fills 1 KiB of LDS without passing
// through registers.  Issued from inline asm so that the compiler does not wait for it before
// every LDS read; completion is tracked by explicit vmcnt waits before the barrier that
// publishes a stage.  Addressed as a 64-bit scalar base plus a 32-bit per-lane offset.
// This form expects M0 already set and sets M0 to the LDS address of the next LDS-DMA
// afterwards, so the MFMAs issued in between cover the M0 -> LDS-DMA hazard.  The compiler does not use M0 on gfx950 (LDS instructions do
// not read it), so keeping it live between statements is safe.
__device__ __forceinline__ void lds_dma16_next(uint32_t voff, const void* sbase, uint32_t next_lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1\n\ts_mov_b32 m0, %2" ::"v"(voff), "s"(sbase), "s"(next_lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void set_m0(uint32_t lds_addr) { asm volatile("s_mov_b32 m0, %0" ::"s"(lds_addr) : "m0"); }
// The dword forms of the two above (lane l writes LDS m0 + 4 l): block exponents of FP4 rows.
__device__ __forceinline__ void lds_dma4_next(uint32_t voff, const void* sbase, uint32_t next_lds) {
    asm volatile("global_load_lds_dword %0, %1\n\ts_mov_b32 m0, %2" ::"v"(voff), "s"(sbase), "s"(next_lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_s(uint32_t lds_addr, uint32_t voff, const void* sbase) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds_addr), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_dma16_s(uint32_t lds_addr, uint32_t voff, const void* sbase) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<T*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

}  // namespace qdt
