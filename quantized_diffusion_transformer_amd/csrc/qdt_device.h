// Device-side helpers shared by the HIP kernels: bf16 conversion and the epilogue
// arithmetic.  The fused GEMM epilogue and the split-K epilogue call the same functions,
// so an output element gets the same fp32 operation sequence whichever plan ran.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qdt {

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

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

// Gated SiLU of the fused FFN epilogue: (g / (1 + exp(-g))) * u, for 4 outputs.
// (Serving sub-second Ideogram v4 without quality loss, fused-epilogue paragraph.)
// The result is rounded to bf16 (relative half-ulp 2^-9), so the hardware exp2 and reciprocal
// (about 1 fp32 ulp each) are used: for |g| <= 64 the relative error of s * u stays below
// about 4e-6 (the rounding of -g * log2(e) dominates), which can move a bf16 rounding by at
// most one ulp.  Elements with |g| > 64 take the correctly rounded expf and division (so the
// tiny sigmoid tail never underflows or flushes); the choice is per element, the branch only
// skips that code when no lane needs it.
__device__ __forceinline__ float silu_fast(float g) {
    const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ void silu_gate4(const float (&g)[4], const float (&u)[4], float (&y)[4]) {
    float s[4];
    bool big = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        s[r] = silu_fast(g[r]);
        big |= __builtin_fabsf(g[r]) > 64.0f;
    }
    if (big) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (__builtin_fabsf(g[r]) > 64.0f) s[r] = g[r] / (1.0f + expf(-g[r]));
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = s[r] * u[r];
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

__device__ __forceinline__ double wave_sum64(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace qdt
