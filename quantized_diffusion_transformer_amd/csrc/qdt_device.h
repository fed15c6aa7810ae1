// Device-side helpers shared by the HIP kernels: bf16 conversion and the epilogue
// arithmetic.  The fused GEMM epilogue and the split-K epilogue call the same functions,
// so an output element gets the same fp32 operation sequence whichever plan ran.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qdt {

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Round-half-to-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

// Two round-half-to-even conversions in one v_cvt_pk_bf16_f32; lo in bits 0..15.
typedef float qdt_v2f __attribute__((ext_vector_type(2)));
typedef __bf16 qdt_v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const qdt_v2bf r = __builtin_convertvector((qdt_v2f){lo, hi}, qdt_v2bf);
    return __builtin_bit_cast(uint32_t, r);
}

// Dequantization + bias of one accumulator: fmaf((float)acc, sx * sw, b).
// (Quantizing a Dual-Branch Flow-Matching DiT for Consumer GPUs, W8A8 recipe: per-token
// activation scale times per-output-row weight scale; the fused multiply-add order is the
// reading fixed for this library.)
__device__ __forceinline__ float dequant(int32_t acc, float sx, float sw, float b) {
    float d = sx * sw;
    return __builtin_fmaf((float)acc, d, b);
}

// Gated SiLU of the fused FFN epilogue: (g / (1 + exp(-g))) * u.
// (Serving sub-second Ideogram v4 without quality loss, fused-epilogue paragraph.)
__device__ __forceinline__ float silu_gate(float g, float u) {
    float e = expf(-g);
    float den = 1.0f + e;
    float s = g / den;
    return s * u;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace qdt
