// Row and column kernels of the W8A8 linear: calibration max-abs, the smoothing vector and
// the per-row symmetric INT8 quantizer (per token for activations, per output row for the
// smoothed weights).
//
// Method: "Quantizing a Dual-Branch Flow-Matching Diffusion Transformer for Consumer GPUs"
// (INT8 and GGUF PTQ of Ideogram 4.0), W8A8 recipe paragraph -- per-token dynamic INT8
// activations, per-output-row INT8 weights, SmoothQuant lambda_j = s_j^a / max_i|W_ij|^(1-a)
// with a = 0.5, activations scaled down by lambda and weights up.
//
// The quantizer is HBM-bound: one read of the bf16 row, one write of the int8 row.  A row is
// owned by one wavefront (K <= 8192) or one workgroup (larger K) and held in registers
// between the max-abs reduction and the quantization, so X is read once.
#include <atomic>

#include "qdt_device.h"
#include "qdt_internal.h"

namespace qdt {

// ---------------------------------------------------------------------------- fill
__global__ void fill_f32_kernel(float* __restrict__ p, float v, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, v, n);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- column max-abs
// Block: 4 waves; each lane owns 8 consecutive columns of a 512-column window; waves stride
// over a chunk of rows; the 4 partial maxima meet in LDS and one atomic max per column
// (fp32 bit patterns of non-negative values order like unsigned integers) merges blocks.
constexpr int kColmaxRows = 64;

__global__ __launch_bounds__(256) void colmax_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                     int64_t ldx, float* __restrict__ s) {
    __shared__ float part[4][512];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t j0 = (int64_t)blockIdx.x * 512 + lane * 8;
    const int64_t r0 = (int64_t)blockIdx.y * kColmaxRows;
    const int64_t r1 = min(M, r0 + kColmaxRows);
    float mx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mx[e] = 0.0f;
    if (j0 < K) {
        for (int64_t r = r0 + wave; r < r1; r += 4) {
            uint4 raw = *reinterpret_cast<const uint4*>(X + r * ldx + j0);
            uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                mx[2 * e] = fmaxf(mx[2 * e], fabsf(bf16_to_f32(w[e] & 0xFFFFu)));
                mx[2 * e + 1] = fmaxf(mx[2 * e + 1], fabsf(bf16_to_f32(w[e] >> 16)));
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[wave][lane * 8 + e] = mx[e];
    __syncthreads();
    for (int c = threadIdx.x; c < 512; c += 256) {
        int64_t j = (int64_t)blockIdx.x * 512 + c;
        if (j < K) {
            float v = fmaxf(fmaxf(part[0][c], part[1][c]), fmaxf(part[2][c], part[3][c]));
            atomicMax(reinterpret_cast<unsigned int*>(s + j), __float_as_uint(v));
        }
    }
}

hipError_t launch_colmax(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, float* s, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    dim3 grid((unsigned)((K + 511) / 512), (unsigned)((M + kColmaxRows - 1) / kColmaxRows));
    hipLaunchKernelGGL(colmax_kernel, grid, dim3(256), 0, st, X, M, K, ldx, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- lambda
// lam_inout holds w_j = max_n |W_nj| on entry and lambda_j on exit.
__global__ void lambda_kernel(const float* __restrict__ s, float* __restrict__ lam, float* __restrict__ inv,
                              int64_t K, float alpha, int half) {
    int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= K) return;
    float sj = s[j], wj = lam[j];
    float l;
    if (sj == 0.0f || wj == 0.0f)
        l = 1.0f;
    else if (half)
        l = sqrtf(sj) / sqrtf(wj);
    else
        l = powf(sj, alpha) / powf(wj, 1.0f - alpha);
    lam[j] = l;
    inv[j] = 1.0f / l;
}

hipError_t launch_lambda(const float* s, float* lam, float* inv, int64_t K, float alpha, hipStream_t st) {
    int64_t blocks = (K + 255) / 256;
    hipLaunchKernelGGL(lambda_kernel, dim3((unsigned)blocks), dim3(256), 0, st, s, lam, inv, K, alpha,
                       alpha == 0.5f ? 1 : 0);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- per-row INT8
// q = clamp(rint(v / scale), -127, 127) with scale = max|v| / 127, bit-exact, without a
// division per element:
//   * rcp = RN(1 / scale), t = RN(v * rcp).  For |v / scale| <= 127 the two roundings keep
//     |t - v / scale| < 2^-16.
//   * m = RN(t + 1.5 * 2^23) rounds t to the nearest integer (ties to even): for |t| < 2^22 the
//     sum's ulp is 1, and the integer sits in the low mantissa bits, so the low byte of m is the
//     two's-complement int8 of rint(t) (|t| <= 127.001 here, so no clamp is needed).
//   * If t is at least 2^-15 away from every half-integer, v / scale and RN(v / scale) lie on the
//     same side of the same half-integers as t, so rint(t) == rint(RN(v / scale)).  The test is
//     |t - rint(t)| < 0.5 - 2^-15.  Chunks where some element fails it (probability about 6e-5
//     per element) are redone with the correctly rounded division, as are rows whose scale is
//     below FLT_MIN (1 / scale overflows).
constexpr float kRoundMagic = 12582912.0f;          // 1.5 * 2^23
constexpr float kNearTie = 0.5f - 3.0517578125e-05f;  // 0.5 - 2^-15

__device__ __forceinline__ int quant_exact(float v, float sc) {
    const float q = fminf(fmaxf(rintf(v / sc), -127.0f), 127.0f);
    return (int)q;
}

// A 16-byte load of activations, which these kernels read exactly once: non-temporal, so the
// stream does not displace what the next kernel reads (the weights and the quantized X, from L2
// and the Infinity Cache).  Measured on the 4608 x 4608 quantize pass: 17.0 -> 14.3 us, and the
// quantize + linear step 92.7 -> 91.1 us; the fused adaLN 25.1 -> 25.0 us (4608 rows) and 60.5 -> 59.8 us
// (16896 rows).  The FP4 quantizer keeps plain loads (its 4608 x 4608 step measured 1 us slower).
__device__ __forceinline__ uint4 load_once16(const uint16_t* p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Chunk j of a row (8 elements), zero past the row's end (j >= nch).  The load is issued for every
// lane (lanes past the end re-read the row's last chunk) and the zero is a select: with the load
// under a branch, the compiler copied each loaded value inside its branch and so waited for every
// load before issuing the next, serializing a row's C loads.
__device__ __forceinline__ uint4 load_row_chunk(const uint16_t* row, int64_t j, int64_t nch) {
    const uint4 v = load_once16(row + min(j, nch - 1) * 8);
    return j < nch ? v : make_uint4(0u, 0u, 0u, 0u);
}

// bytes 0 of a, b, c, d -> one dword (a in byte 0)
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// One row per wave (WPR == 1, 4 waves per block) or per block of WPR waves; C chunks of 8
// consecutive elements per lane (chunk index lane + 64 c within the row, or thread + 64 WPR c).
// Rows are grid-strided.  With WPR == 1 (K <= 8192) the column multipliers are staged in LDS
// once per block and shared by the rows of its 4 waves; larger K reads them per row (L2 hits).
constexpr int kQuantMaxLdsK = 8192;

template <int WPR, int C>
__global__ __launch_bounds__(WPR == 1 ? 256 : WPR * 64) void quant_rows_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const float* __restrict__ colmul, int64_t M, int64_t K,
    int8_t* __restrict__ Q, float* __restrict__ scale) {
    constexpr int NT = WPR * 64;
    constexpr bool LDSMUL = WPR == 1;
    __shared__ float red[2][WPR > 1 ? WPR : 1];
    extern __shared__ __attribute__((aligned(16))) float smul[];  // K floats when LDSMUL and colmul
    const int lane = threadIdx.x & 63;
    const int t = WPR == 1 ? lane : (int)threadIdx.x;
    // the row is uniform per wave (WPR == 1) or per block
    const int64_t row0 = WPR == 1 ? (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)
                                  : (int64_t)blockIdx.x;
    const int64_t rstep = WPR == 1 ? (int64_t)gridDim.x * 4 : (int64_t)gridDim.x;
    const int64_t nch = K >> 3;
    if (LDSMUL && colmul) {
        for (int64_t j = threadIdx.x; j < nch * 2; j += blockDim.x)
            *reinterpret_cast<float4*>(smul + j * 4) = *reinterpret_cast<const float4*>(colmul + j * 4);
        __syncthreads();
    }
    // multipliers of chunk j (8 columns)
    auto load_mul = [&](int64_t j, float (&mm)[8]) __attribute__((always_inline)) {
        const float* src = LDSMUL ? smul + j * 8 : colmul + j * 8;
        const float4 m0 = *reinterpret_cast<const float4*>(src);
        const float4 m1 = *reinterpret_cast<const float4*>(src + 4);
        mm[0] = m0.x; mm[1] = m0.y; mm[2] = m0.z; mm[3] = m0.w;
        mm[4] = m1.x; mm[5] = m1.y; mm[6] = m1.z; mm[7] = m1.w;
    };

    // Four waves per row (K in (8192, 16384]) keep the row's values in registers and load the
    // block's next row once this row's max is known: the second pass loads nothing, so those loads
    // overlap it (4608 x 12288: 38.2 -> 35.9 us).  With 16 waves per row the extra registers spill
    // at the 128-register cap, and the 512 x 53248 step measured no faster.
    constexpr bool PF = WPR == 4 && C <= 12;
    // Loads of chunks past the row's end: under a branch (zero without a load) or clamped into the
    // row (load_row_chunk).  With 16 chunks per lane the branch form made the compiler serialize the
    // row's loads (a copy of each loaded value inside its branch waits for it): clamped, 4608 x 8192
    // measured 34.3 -> 26.7 us with identical outputs.  Elsewhere the branch form keeps the loads back
    // to back with fewer registers (9 chunks: 107 against 123 VGPRs), or measured faster anyway (four
    // waves per row, which serializes 4 of its loads: 36.0 against 38.7 us at 4608 x 12288).
    constexpr bool CLAMP = WPR == 1 && C == 16;
    auto chunk_load = [&](const uint16_t* rowp, int64_t j) __attribute__((always_inline)) {
        if constexpr (CLAMP)
            return load_row_chunk(rowp, j, nch);
        else
            return j < nch ? load_once16(rowp + j * 8) : make_uint4(0u, 0u, 0u, 0u);
    };
    uint4 nxt[PF ? C : 1];
    if constexpr (PF) {
        if (row0 < M) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int64_t j = t + (int64_t)c * NT;
                nxt[c] = chunk_load(X + row0 * ldx, j);
            }
        }
    }
    int parity = 0;
    for (int64_t row = row0; row < M; row += rstep, parity ^= 1) {
        const uint16_t* x = X + row * ldx;
        uint4 raw[C];
        if constexpr (PF) {
#pragma unroll
            for (int c = 0; c < C; ++c) raw[c] = nxt[c];
        } else {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int64_t j = t + (int64_t)c * NT;
                raw[c] = chunk_load(x, j);
            }
        }
        // v = bf16 element * multiplier; chunk c, computed again in the second pass when the
        // row does not fit in registers as fp32 (C > 12)
        auto chunk_vals = [&](int c, float (&vc)[8]) __attribute__((always_inline)) {
            const uint32_t w[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vc[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
                vc[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
            const int64_t j = t + (int64_t)c * NT;
            if (colmul && j < nch) {
                float mm[8];
                load_mul(j, mm);
#pragma unroll
                for (int e = 0; e < 8; ++e) vc[e] *= mm[e];
            }
        };
        constexpr bool KEEP = C <= 12;
        float v[KEEP ? C : 1][8];
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            float vc[8];
            chunk_vals(c, vc);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                amax = fmaxf(amax, fabsf(vc[e]));
                if constexpr (KEEP) v[c][e] = vc[e];
            }
            // without these empty asm statements the compiler keeps every chunk's values live
            // into the second pass (295 VGPRs at C = 16, 315 spills with 16 waves per row)
            if constexpr (!KEEP) asm volatile("" : "+v"(amax));
        }
        if constexpr (!KEEP) {
#pragma unroll
            for (int c = 0; c < C; ++c) asm volatile("" : "+v"(raw[c].x), "+v"(raw[c].y), "+v"(raw[c].z), "+v"(raw[c].w));
        }
        amax = wave_max(amax);
        if (WPR > 1) {
            // double-buffered across rows: a wave may start the next row while others still
            // read this row's slot
            if (lane == 0) red[parity][threadIdx.x >> 6] = amax;
            __syncthreads();
            amax = red[parity][0];
#pragma unroll
            for (int w = 1; w < WPR; ++w) amax = fmaxf(amax, red[parity][w]);
        }
        if constexpr (PF) {
            const int64_t rn = row + rstep;
            if (rn < M) {
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const int64_t j = t + (int64_t)c * NT;
                    nxt[c] = chunk_load(X + rn * ldx, j);
                }
            }
        }
        const float sc = amax / 127.0f;  // correctly rounded; 0 for an all-zero row
        if (t == 0) scale[row] = sc;
        int8_t* q = Q + row * K;
        if (amax == 0.0f) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int64_t j = t + (int64_t)c * NT;
                if (j < nch) *reinterpret_cast<uint2*>(q + j * 8) = make_uint2(0u, 0u);
            }
            continue;
        }
        const bool fast = sc >= 1.17549435e-38f;
        const float rcp = 1.0f / sc;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t j = t + (int64_t)c * NT;
            float vc[8];
            if constexpr (KEEP) {
#pragma unroll
                for (int e = 0; e < 8; ++e) vc[e] = v[c][e];
            } else {
                chunk_vals(c, vc);
            }
            uint32_t b[8];
            bool near = !fast;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float tq = vc[e] * rcp;
                const float m = tq + kRoundMagic;
                const float r = m - kRoundMagic;
                near |= fabsf(tq - r) >= kNearTie;
                b[e] = __float_as_uint(m);
            }
            if (near) {
#pragma unroll
                for (int e = 0; e < 8; ++e) b[e] = (uint32_t)quant_exact(vc[e], sc);
            }
            if (j < nch)
                *reinterpret_cast<uint2*>(q + j * 8) =
                    make_uint2(pack_low_bytes(b[0], b[1], b[2], b[3]), pack_low_bytes(b[4], b[5], b[6], b[7]));
        }
    }
}

// Grid: at most as many blocks as can be resident at once (occupancy query); rows are
// grid-strided over them.  More waves in flight measured faster than an even row split.
template <int WPR, int C>
static hipError_t launch_quant_cfg(const uint16_t* X, int64_t ldx, const float* colmul, int64_t M, int64_t K,
                                   int8_t* Q, float* scale, hipStream_t st) {
    static_assert(WPR > 1 || C * 64 * 8 <= kQuantMaxLdsK, "column multipliers fit in LDS");
    const int threads = WPR == 1 ? 256 : WPR * 64;
    const size_t lds = (WPR == 1 && colmul) ? (size_t)K * sizeof(float) : 0;
    // cached per configuration (one architecture per process), for the largest LDS request of the
    // configuration (K = 512 C); concurrent first calls compute the same value
    static std::atomic<int> per_cu_cache[2] = {0, 0};
    int per_cu = per_cu_cache[lds ? 1 : 0].load(std::memory_order_relaxed);
    if (per_cu == 0) {
        int v = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, quant_rows_kernel<WPR, C>, threads,
                                                                    lds ? (size_t)C * 512 * sizeof(float) : 0);
        if (e != hipSuccess) return e;
        per_cu = max(v, 1);
        per_cu_cache[lds ? 1 : 0].store(per_cu, std::memory_order_relaxed);
    }
    const int64_t units = WPR == 1 ? (M + 3) / 4 : M;  // blocks for one row per wave
    const int64_t blocks = min(units, (int64_t)per_cu * kNumCU);
    hipLaunchKernelGGL((quant_rows_kernel<WPR, C>), dim3((unsigned)blocks), dim3(threads), lds, st, X, ldx, colmul,
                       M, K, Q, scale);
    return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* X, int64_t ldx, const float* colmul, int64_t M, int64_t K, int8_t* Q,
                             float* scale, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    const int64_t nch = K / 8;  // 16-byte chunks per row
    if (nch <= 64 * 1) return launch_quant_cfg<1, 1>(X, ldx, colmul, M, K, Q, scale, st);
    if (nch <= 64 * 2) return launch_quant_cfg<1, 2>(X, ldx, colmul, M, K, Q, scale, st);
    if (nch <= 64 * 4) return launch_quant_cfg<1, 4>(X, ldx, colmul, M, K, Q, scale, st);
    if (nch <= 64 * 6) return launch_quant_cfg<1, 6>(X, ldx, colmul, M, K, Q, scale, st);
    if (nch <= 64 * 9) return launch_quant_cfg<1, 9>(X, ldx, colmul, M, K, Q, scale, st);
    if (nch <= 64 * 12) return launch_quant_cfg<1, 12>(X, ldx, colmul, M, K, Q, scale, st);
    if (nch <= 64 * 16) return launch_quant_cfg<1, 16>(X, ldx, colmul, M, K, Q, scale, st);
    if (nch <= 256 * 8) return launch_quant_cfg<4, 8>(X, ldx, colmul, M, K, Q, scale, st);
    if (nch <= 1024 * 7) return launch_quant_cfg<16, 7>(X, ldx, colmul, M, K, Q, scale, st);
    return launch_quant_cfg<16, 16>(X, ldx, colmul, M, K, Q, scale, st);
}

// ---------------------------------------------------------------------------- adaLN + INT8
// Producer-fused quantization: the adaptive LayerNorm in front of a quantized linear of a DiT
// block, with the per-token quantizer of that linear's input in the same pass over the row.
// ("Quantizing a Dual-Branch Flow-Matching DiT", related work: the adaLN modulation is
// generated at run time; "Serving sub-second Ideogram v4", fused-epilogue paragraph: the
// small op next to a large one belongs in the same kernel, without a round trip to memory.)
//   mean = sum_j x_j / K,  var = sum_j (x_j - mean)^2 / K
//   r = 1 / sqrtf(var + eps),  n_j = (x_j - mean) * r,  h_j = bf16(n_j * (1 + scale_j) + shift_j)
//   v_j = h_j * inv_lambda_j,  x_scale = max |v| / 127,  q_j = rne(v_j / x_scale) clamped to +-127
// mean and var: sum x and sum x^2 in fp64 (one pass), var = sum x^2 / K - mean^2, both rounded
// to fp32.  The fp64 rounding errors stay far below the fp32 rounding of the results, so these
// are the correctly rounded fp32 statistics except on rare near-ties, whatever the order.
// One wave per row (K <= 8192).  The block stages inv_lambda (1 when absent), 1 + scale and
// shift (0 when absent) as fp32 in LDS, 12 K bytes; 1 + scale is rounded exactly as in the
// definition.  The row stays in registers from the load to the last store: X is read once, Xq
// (and H on request) written once.  The kernel is bound by VALU issue more than by HBM (about 25
// operations per element), so the launch balances rows per SIMD: at most one block per compute
// unit (16 waves, 4 per SIMD; 8 waves where the row needs more registers), each block a
// contiguous run of floor or ceil(M / blocks) rows, taken by its waves in turn.  At 4608 rows
// that is 18 rows per block and at most 5 per SIMD (a grid-stride launch of 8-wave blocks left
// 6 on some SIMDs).  Every wave issues its first row's loads at once: a stagger of the one-row
// waves' first loads (so that the two-row waves' rows arrive first) helped while each wave's loads
// ran one after another, and measured slower once they went out back to back (4608 rows 21.5 ->
// 20.8 us without it).
constexpr int adaln_waves(int C) { return C <= 9 ? 16 : 8; }

template <int C, bool QUANT>
__global__ __launch_bounds__(adaln_waves(C) * 64) void adaln_quant_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const uint16_t* __restrict__ shift,
    const uint16_t* __restrict__ scale, float eps, const float* __restrict__ colmul, int64_t M, int64_t K,
    int8_t* __restrict__ Q, float* __restrict__ xscale, uint16_t* __restrict__ H, int64_t rq, int64_t rr) {
    extern __shared__ __attribute__((aligned(16))) float smem_f[];
    float* smul = smem_f;      // K: inv_lambda
    float* sg = smem_f + K;    // K: 1 + scale
    float* sb = sg + K;        // K: shift
    const int lane = threadIdx.x & 63;
    const int64_t nch = K >> 3;
    for (int64_t j = threadIdx.x; j < nch; j += blockDim.x) {
        float4 m0 = make_float4(1.0f, 1.0f, 1.0f, 1.0f), m1 = m0;
        if (colmul) {
            m0 = *reinterpret_cast<const float4*>(colmul + j * 8);
            m1 = *reinterpret_cast<const float4*>(colmul + j * 8 + 4);
        }
        *reinterpret_cast<float4*>(smul + j * 8) = m0;
        *reinterpret_cast<float4*>(smul + j * 8 + 4) = m1;
        const uint4 sc = scale ? *reinterpret_cast<const uint4*>(scale + j * 8) : make_uint4(0u, 0u, 0u, 0u);
        const uint4 sh = shift ? *reinterpret_cast<const uint4*>(shift + j * 8) : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t scw[4] = {sc.x, sc.y, sc.z, sc.w}, shw[4] = {sh.x, sh.y, sh.z, sh.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            sg[j * 8 + 2 * p] = 1.0f + bf16_to_f32(scw[p] & 0xFFFFu);
            sg[j * 8 + 2 * p + 1] = 1.0f + __uint_as_float(scw[p] & 0xFFFF0000u);
            sb[j * 8 + 2 * p] = bf16_to_f32(shw[p] & 0xFFFFu);
            sb[j * 8 + 2 * p + 1] = __uint_as_float(shw[p] & 0xFFFF0000u);
        }
    }
    __syncthreads();
    auto lds8 = [&](const float* base, int64_t j, float (&o)[8]) __attribute__((always_inline)) {
        const float4 a = *reinterpret_cast<const float4*>(base + j * 8);
        const float4 b = *reinterpret_cast<const float4*>(base + j * 8 + 4);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    };
    // rows [rb0, rb1) of this block: rq each, one more for the first rr blocks
    constexpr int W = adaln_waves(C);
    const int64_t rb0 = (int64_t)blockIdx.x * rq + min((int64_t)blockIdx.x, rr);
    const int64_t rb1 = rb0 + rq + ((int64_t)blockIdx.x < rr ? 1 : 0);
    for (int64_t row = rb0 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); row < rb1; row += W) {
        const uint16_t* x = X + row * ldx;
        uint4 raw[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t j = lane + (int64_t)c * 64;
            // every chunk is loaded (lanes past the row re-read its last chunk, skipped below), so
            // the row's loads go out back to back: under a branch, or with the zero as a select
            // right after each load, the compiler waited for each load before issuing the next
            raw[c] = load_once16(x + min(j, nch - 1) * 8);
        }
        // element e of chunk c (bf16 pairs, low half first)
        auto elem = [&](int c, int e) __attribute__((always_inline)) {
            const uint32_t ww[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
            return (e & 1) ? __uint_as_float(ww[e >> 1] & 0xFFFF0000u) : bf16_to_f32(ww[e >> 1] & 0xFFFFu);
        };
        // statistics over the row's chunks
        double s1 = 0.0, s2 = 0.0;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (lane + (int64_t)c * 64 >= nch) continue;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double v = (double)elem(c, e);
                s1 += v;
                s2 = __builtin_fma(v, v, s2);
            }
        }
        s1 = wave_sum64(s1);
        s2 = wave_sum64(s2);
        const double mean64 = s1 / (double)K;
        const double var64 = __builtin_fmax(__builtin_fma(-mean64, mean64, s2 / (double)K), 0.0);
        const float mean = (float)mean64;
        const float r = 1.0f / sqrtf((float)var64 + eps);
        // Each pass converts the packed row again (one shift or mask per element) instead of
        // keeping 8 C fp32 values live across passes: an empty asm that "modifies" the packed
        // registers stops the compiler from reusing conversions of the statistics pass.
#pragma unroll
        for (int c = 0; c < C; ++c) asm volatile("" : "+v"(raw[c].x), "+v"(raw[c].y), "+v"(raw[c].z), "+v"(raw[c].w));
        // h = bf16(n * (1 + scale) + shift); v = h * inv_lambda
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t j = lane + (int64_t)c * 64;
            if (j >= nch) continue;
            float g[8], bb[8], mm[8];
            lds8(sg, j, g);
            lds8(sb, j, bb);
            if constexpr (QUANT) lds8(smul, j, mm);
            uint32_t hp[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float h0 = ((elem(c, 2 * p) - mean) * r) * g[2 * p] + bb[2 * p];
                const float h1 = ((elem(c, 2 * p + 1) - mean) * r) * g[2 * p + 1] + bb[2 * p + 1];
                hp[p] = pack_bf16x2(h0, h1);
            }
            raw[c] = make_uint4(hp[0], hp[1], hp[2], hp[3]);
            if (H) *reinterpret_cast<uint4*>(H + row * K + j * 8) = raw[c];
            if constexpr (QUANT) {
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(elem(c, e) * mm[e]));
            }
        }
        if constexpr (!QUANT) continue;
        amax = wave_max(amax);
        const float sc = amax / 127.0f;
        if (lane == 0) xscale[row] = sc;
        int8_t* q = Q + row * K;
        const bool fast = sc >= 1.17549435e-38f;
        const float rcp = 1.0f / sc;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t j = lane + (int64_t)c * 64;
            if (j >= nch) continue;
            if (amax == 0.0f) {
                *reinterpret_cast<uint2*>(q + j * 8) = make_uint2(0u, 0u);
                continue;
            }
            // v again from the packed h (keeping 8 C fp32 values live instead measured slower:
            // fewer waves per SIMD)
            float vc[8], mm[8];
            lds8(smul, j, mm);
#pragma unroll
            for (int e = 0; e < 8; ++e) vc[e] = elem(c, e) * mm[e];
            // the largest distance to the nearest integer decides the chunk's path (one max per
            // element instead of a compare and a flag)
            uint32_t b[8];
            float dmax = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float tq = vc[e] * rcp;
                const float m = tq + kRoundMagic;
                dmax = fmaxf(dmax, fabsf(tq - (m - kRoundMagic)));
                b[e] = __float_as_uint(m);
            }
            if (!fast || dmax >= kNearTie) {
#pragma unroll
                for (int e = 0; e < 8; ++e) b[e] = (uint32_t)quant_exact(vc[e], sc);
            }
            *reinterpret_cast<uint2*>(q + j * 8) =
                make_uint2(pack_low_bytes(b[0], b[1], b[2], b[3]), pack_low_bytes(b[4], b[5], b[6], b[7]));
        }
    }
}

template <int C, bool QUANT>
static hipError_t launch_adaln_cfg(const uint16_t* X, int64_t ldx, const uint16_t* shift, const uint16_t* scale,
                                   float eps, const float* colmul, int64_t M, int64_t K, int8_t* Q, float* xscale,
                                   uint16_t* H, hipStream_t st) {
    const int threads = adaln_waves(C) * 64;
    const size_t lds = (size_t)K * 12;
    // cached like launch_quant_cfg's, for the largest LDS request of the configuration (K = 512 C)
    static std::atomic<int> per_cu_cache{0};
    int per_cu = per_cu_cache.load(std::memory_order_relaxed);
    if (per_cu == 0) {
        int v = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, adaln_quant_kernel<C, QUANT>, threads,
                                                                    (size_t)C * 512 * 12);
        if (e != hipSuccess) return e;
        per_cu = max(v, 1);
        per_cu_cache.store(per_cu, std::memory_order_relaxed);
    }
    const int64_t units = (M + adaln_waves(C) - 1) / adaln_waves(C);
    const int64_t blocks = min(units, (int64_t)per_cu * kNumCU);
    hipLaunchKernelGGL((adaln_quant_kernel<C, QUANT>), dim3((unsigned)blocks), dim3(threads), lds, st, X, ldx, shift,
                       scale, eps, colmul, M, K, Q, xscale, H, M / blocks, M % blocks);
    return hipGetLastError();
}

template <bool QUANT>
static hipError_t launch_adaln(const uint16_t* X, int64_t ldx, const uint16_t* shift, const uint16_t* scale, float eps,
                               const float* colmul, int64_t M, int64_t K, int8_t* Q, float* xscale, uint16_t* H,
                               hipStream_t st) {
    const int64_t nch = K / 8;
    if (nch <= 64 * 1) return launch_adaln_cfg<1, QUANT>(X, ldx, shift, scale, eps, colmul, M, K, Q, xscale, H, st);
    if (nch <= 64 * 2) return launch_adaln_cfg<2, QUANT>(X, ldx, shift, scale, eps, colmul, M, K, Q, xscale, H, st);
    if (nch <= 64 * 4) return launch_adaln_cfg<4, QUANT>(X, ldx, shift, scale, eps, colmul, M, K, Q, xscale, H, st);
    if (nch <= 64 * 6) return launch_adaln_cfg<6, QUANT>(X, ldx, shift, scale, eps, colmul, M, K, Q, xscale, H, st);
    if (nch <= 64 * 9) return launch_adaln_cfg<9, QUANT>(X, ldx, shift, scale, eps, colmul, M, K, Q, xscale, H, st);
    if (nch <= 64 * 12) return launch_adaln_cfg<12, QUANT>(X, ldx, shift, scale, eps, colmul, M, K, Q, xscale, H, st);
    return launch_adaln_cfg<16, QUANT>(X, ldx, shift, scale, eps, colmul, M, K, Q, xscale, H, st);
}

hipError_t launch_adaln_quant(const uint16_t* X, int64_t ldx, const uint16_t* shift, const uint16_t* scale, float eps,
                              const float* colmul, int64_t M, int64_t K, int8_t* Q, float* xscale, uint16_t* H,
                              hipStream_t st) {
    if (M <= 0) return hipSuccess;
    if (Q) return launch_adaln<true>(X, ldx, shift, scale, eps, colmul, M, K, Q, xscale, H, st);
    return launch_adaln<false>(X, ldx, shift, scale, eps, colmul, M, K, Q, xscale, H, st);
}

// ---------------------------------------------------------------------------- block-scaled FP4
// MXFP4, the block-scaled 4-bit floating point native to the MI355X matrix cores ("Serving
// sub-second Ideogram v4 without quality loss": the DiT runs in a block-scaled 4-bit float on the
// authors' GPUs).  Per block of 32 consecutive elements of a row (v = x * colmul):
//   e = clamp(floor(log2(max |v|)) - 2, -127, 127)   (-127 for an all-zero block), byte e + 127
//   code = fp4(v / 2^e): nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to mantissa 0, saturating at
//          6; sign << 3 | index, zero stored as +0; two codes per byte, even element low.
// One lane converts 8 consecutive elements (16 bytes of bf16), so a block is a quad of lanes;
// the quad max takes two lane exchanges.  v / 2^e is exact (v_ldexp_f32) and lies in (-8, 8);
// v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds it to the nearest code with ties to even and
// saturates, as the definition reads, except that it keeps the sign of values that round to
// zero, which is cleared afterwards.  Bytes per element: 2 read, 0.5 + 1/32 written.
__global__ __launch_bounds__(256) void mx_quant_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                       const float* __restrict__ colmul, int64_t M, int64_t K,
                                                       uint8_t* __restrict__ Q, uint8_t* __restrict__ S) {
    const int64_t cpr = K >> 3;  // 8-element chunks per row
    const int64_t total = M * cpr;
    const int lane = threadIdx.x & 63;
    for (int64_t base = ((int64_t)blockIdx.x * blockDim.x + (threadIdx.x & ~63)); base < total;
         base += (int64_t)gridDim.x * blockDim.x) {
        const int64_t c = base + lane;  // quads of lanes are blocks: cpr % 4 == 0 and base % 64 == 0
        const bool ok = c < total;
        const int64_t row = ok ? c / cpr : 0, cc = ok ? c % cpr : 0;
        float v[8];
        const uint4 raw = ok ? *reinterpret_cast<const uint4*>(X + row * ldx + cc * 8) : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
            v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
        if (colmul && ok) {
            const float4 m0 = *reinterpret_cast<const float4*>(colmul + cc * 8);
            const float4 m1 = *reinterpret_cast<const float4*>(colmul + cc * 8 + 4);
            const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= mm[e];
        }
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
        // amax = f * 2^ex with f in [0.5, 1): floor(log2 amax) = ex - 1
        int ex = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) - 3 : -127;
        ex = min(max(ex, -127), 127);
        float t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = __builtin_ldexpf(v[e], -ex);
        uint32_t packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, t[0], t[1], 1.0f, 0);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, t[2], t[3], 1.0f, 1);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, t[4], t[5], 1.0f, 2);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, t[6], t[7], 1.0f, 3);
        // clear the sign of zero magnitudes: a nibble keeps bit 3 only if its low 3 bits are nonzero
        const uint32_t mag = packed & 0x77777777u;
        packed &= 0x77777777u | ((mag + 0x77777777u) & 0x88888888u);
        if (ok) {
            *reinterpret_cast<uint32_t*>(Q + row * (K >> 1) + cc * 4) = packed;
            // stage-major exponents: block b of the row goes to group b / 8 (256 elements), byte
            // 2 (b % 4) + (b % 8) / 4 of the row's 8-byte slot in that group
            if ((lane & 3) == 0) {
                const int64_t b = cc >> 2, w = b & 7;
                S[(b >> 3) * M * 8 + row * 8 + 2 * (w & 3) + (w >> 2)] = (uint8_t)(ex + 127);
            }
        }
    }
}

hipError_t launch_mx_quant(const uint16_t* X, int64_t ldx, const float* colmul, int64_t M, int64_t K, uint8_t* Q,
                           uint8_t* S, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    const int64_t chunks = M * (K >> 3);
    const int64_t blocks = min((chunks + 255) / 256, (int64_t)kNumCU * 16);
    hipLaunchKernelGGL(mx_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, st, X, ldx, colmul, M, K, Q, S);
    return hipGetLastError();
}

}  // namespace qdt
