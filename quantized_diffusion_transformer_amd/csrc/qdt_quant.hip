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
// Exact rint(v / scale) from a reciprocal: with rcp = RN(1/scale) and t = RN(v * rcp),
// |t - v/scale| < 2^-16 whenever |v/scale| <= 127 (two roundings of relative size 2^-24).
// If t is farther than 2^-15 from every half-integer, v/scale and its correctly rounded fp32
// quotient lie on the same side of the same half-integers as t, so rint(t) equals
// rint(RN(v / scale)).  Otherwise (probability about 6e-5 per element) the element takes the
// correctly rounded division.  Rows whose scale is below FLT_MIN (1/scale would overflow)
// always take the division.
__device__ __forceinline__ int quant_one(float v, float sc, float rcp, bool fast) {
    float q;
    float t = v * rcp;
    float r = rintf(t);
    if (fast && fabsf(t - r) < 0.5f - 3.0517578125e-05f) {
        q = r;
    } else {
        q = rintf(v / sc);
    }
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    return (int)q;
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)(d & 0xFF) << 24);
}

// WPR waves per row, C chunks of 8 elements per lane.  WPR == 1: 4 rows per 256-thread block.
template <int WPR, int C>
__global__ __launch_bounds__(WPR == 1 ? 256 : WPR * 64) void quant_rows_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const float* __restrict__ colmul, int64_t M, int64_t K,
    int8_t* __restrict__ Q, float* __restrict__ scale) {
    constexpr int NT = WPR * 64;
    __shared__ float red[WPR > 1 ? WPR : 1];
    const int lane = threadIdx.x & 63;
    const int64_t row = WPR == 1 ? (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6) : (int64_t)blockIdx.x;
    const int t = WPR == 1 ? lane : (int)threadIdx.x;
    if (WPR == 1 && row >= M) return;
    const uint16_t* x = X + row * ldx;
    const int64_t nch = K >> 3;

    float v[C][8];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int64_t j = t + (int64_t)c * NT;
        if (j < nch) {
            uint4 raw = *reinterpret_cast<const uint4*>(x + j * 8);
            uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[c][2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
                v[c][2 * e + 1] = bf16_to_f32(w[e] >> 16);
            }
            if (colmul) {
                float4 m0 = *reinterpret_cast<const float4*>(colmul + j * 8);
                float4 m1 = *reinterpret_cast<const float4*>(colmul + j * 8 + 4);
                v[c][0] *= m0.x; v[c][1] *= m0.y; v[c][2] *= m0.z; v[c][3] *= m0.w;
                v[c][4] *= m1.x; v[c][5] *= m1.y; v[c][6] *= m1.z; v[c][7] *= m1.w;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[c][e]));
        }
    }
    amax = wave_max(amax);
    if (WPR > 1) {
        if (lane == 0) red[threadIdx.x >> 6] = amax;
        __syncthreads();
        amax = red[0];
#pragma unroll
        for (int w = 1; w < WPR; ++w) amax = fmaxf(amax, red[w]);
    }
    const float sc = amax / 127.0f;  // correctly rounded; 0 for an all-zero row
    if (t == 0) scale[row] = sc;
    const bool fast = sc >= 1.17549435e-38f;
    const float rcp = fast ? 1.0f / sc : 0.0f;
    int8_t* q = Q + row * K;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int64_t j = t + (int64_t)c * NT;
        if (j < nch) {
            uint2 out;
            if (amax == 0.0f) {
                out = make_uint2(0u, 0u);
            } else {
                int qi[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) qi[e] = quant_one(v[c][e], sc, rcp, fast);
                out.x = pack4(qi[0], qi[1], qi[2], qi[3]);
                out.y = pack4(qi[4], qi[5], qi[6], qi[7]);
            }
            *reinterpret_cast<uint2*>(q + j * 8) = out;
        }
    }
}

template <int WPR, int C>
static hipError_t launch_quant_cfg(const uint16_t* X, int64_t ldx, const float* colmul, int64_t M, int64_t K,
                                   int8_t* Q, float* scale, hipStream_t st) {
    const int64_t blocks = WPR == 1 ? (M + 3) / 4 : M;
    const int threads = WPR == 1 ? 256 : WPR * 64;
    hipLaunchKernelGGL((quant_rows_kernel<WPR, C>), dim3((unsigned)blocks), dim3(threads), 0, st, X, ldx, colmul, M,
                       K, Q, scale);
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

}  // namespace qdt
