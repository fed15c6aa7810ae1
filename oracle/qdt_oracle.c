/*
 * qdt_oracle.c -- plain, slow, obviously correct CPU oracle of the W8A8 DiT linear.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code, header, table or helper
 * with the HIP path; its inputs come from the seeded generator module only.
 *
 * Pages followed (titles as published):
 *   [PTQ]  "Quantizing a Dual-Branch Flow-Matching Diffusion Transformer for Consumer
 *          GPUs: INT8 and GGUF Post-Training Quantization of Ideogram 4.0" --
 *          the W8A8 recipe paragraph of its method section (per-output-row INT8
 *          weights, per-token dynamic INT8 activations, SmoothQuant with alpha = 0.5,
 *          lambda_j = s_j^alpha / max_i |W_ij|^(1-alpha), activations scaled down and
 *          weights scaled up before quantization), and its related-work paragraph
 *          (per-token dynamic activations with per-channel weights).
 *   [FAL]  "Serving sub-second Ideogram v4 without quality loss" -- the paragraph on
 *          fused epilogues: each large matmul is followed by a small op (RMSNorm or
 *          a gated SiLU), and attention heads are 256 wide.
 *   [ZC]   "Faster Ideogram 4 with Less Prompt Compute" -- section "Most of the Tensor
 *          Was Zero": each row goes through the linear on its own, and with the bias
 *          added an all-zero input row comes out as exactly the bias vector.
 *
 * Readings where the pages are silent (each is also listed with the design notes):
 *   - alpha = 0.5 is evaluated as sqrtf(s)/sqrtf(w); lambda = 1 where s or w is 0;
 *     other alpha use powf(s, alpha) / powf(w, 1 - alpha).
 *   - the activation side multiplies by inv_lambda = 1/lambda (computed once).
 *   - symmetric INT8: scale = amax / 127, q = clamp(rint(v / scale), -127, 127), with a
 *     correctly rounded fp32 division and round-half-to-even; an all-zero row has
 *     scale 0 and q = 0.
 *   - BIAS epilogue: y = fmaf((float)acc, sx * sw, bias), then bf16 round-half-even.
 *   - SILU_GATE: rows [gate(0..F-1); up(F..2F-1)], Y = bf16((g / (1 + expf(-g))) * u).
 *   - HEAD_RMSNORM: per row and per head of head_dim columns, ss = sum y^2 (fp64 here),
 *     ms = (float)ss / head_dim, r = 1 / sqrtf(ms + eps), Y = bf16((y * r) * gamma[d]),
 *     one gamma of head_dim entries shared by all heads.
 *   - bf16 GEMM (the protected layer kept unquantized): exact products summed in fp64,
 *     plus bias, rounded to fp32 and then to bf16.
 *   - adaLN before a quantized linear ([PTQ] related work: the modulation is generated at
 *     run time; [FAL]: the small op around a matmul is fused): a LayerNorm over the row
 *     without a learned affine, mean and biased variance summed in fp64 and rounded to fp32,
 *     r = 1 / sqrtf(var + eps), n = (x - mean) * r, h = bf16(n * (1 + scale_j) + shift_j),
 *     with one shift and one scale vector for all rows; h then goes through the per-token
 *     quantizer above.  Parity unpinned by the pages (they do not print the norm); pinned by
 *     closed forms and invariants in the tests.
 *   - Block-scaled 4-bit floating point ([FAL]: the DiT runs in a 4-bit floating-point format
 *     with block scales; the pages name NVFP4 but print none of its parameters): the MXFP4
 *     form native to the target GPU.  Blocks of 32 consecutive elements of a row share a
 *     power-of-two scale 2^e with e = floor(log2(max |v|)) - 2 (the largest element magnitude,
 *     6 = 1.5 * 2^2, has exponent 2), clamped to [-127, 127] and stored biased by 127 in a
 *     byte; e = -127 for an all-zero block.  Each element is v / 2^e rounded to the nearest of
 *     0, 0.5, 1, 1.5, 2, 3, 4, 6 (ties to the even 1-bit mantissa), magnitudes above 6 saturate
 *     to 6, and the 4-bit code is sign << 3 | index with zero always +0.  Two codes per byte,
 *     the even element in the low nibble.  The GEMM sums exact products of the decoded values.
 *   - Weight-only block formats ([PTQ] GGUF paragraph: an 8-bit round-to-nearest format at 8.5
 *     bits per weight, and a 4-bit one at 4.5 bits per weight; [ZC] "The NF4 Exactness
 *     Problem": the text projection multiplies bf16 activations by dequantized weights).  Blocks
 *     of 32 consecutive weights of a row share a 16-bit IEEE half-precision scale
 *     d = half(amax / qmax) (qmax = 127 for 8 bits, 7 for 4 bits; round half to even, half
 *     subnormals kept, magnitudes from 65520 up saturate to 65504), and each weight becomes
 *     q = clamp(rint(w / d), -qmax, qmax) with the fp32 division against the stored scale
 *     (q = 0 when d = 0).  8-bit codes are int8; 4-bit codes are stored as q + 8 in a nibble,
 *     the even element in the low nibble.  The dequantized weight is bf16(q * d) (the product is
 *     exact in fp32), and the GEMM is the bf16 GEMM below on those weights.
 *   - Attention after the QK-norm projection ([FAL]: 256-wide attention heads; the DiT's joint
 *     sequence of text and image tokens): per head h, scaled dot-product softmax attention with
 *     no mask and no positional rotation (the pages print neither), scale 1/sqrt(256) = 1/16:
 *     s_j = (q . k_j) / 16, p_j = exp(s_j - max_j s_j), o = sum_j p_j v_j / sum_j p_j, all in
 *     fp64 from the bf16 inputs, then rounded to fp32 and to bf16.  Q, K, V and O are token-major
 *     [S, ld] with head h in columns 256 h .. 256 h + 255, the layout the projections write.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (no intrinsics, no SIMD pragmas).
 * Floating point: every fp32 operation is IEEE round-to-nearest-even, as written.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_EPI_BIAS 0
#define ORACLE_EPI_SILU_GATE 1
#define ORACLE_EPI_HEAD_RMSNORM 2

static int g_threads = 0;

int oracle_version(void) { return 1; }

void oracle_set_threads(int n) { g_threads = n; }

int oracle_threads(void) {
    if (g_threads > 0) return g_threads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/* ---------------------------------------------------------------- bf16 <-> fp32 */
float oracle_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round-half-to-even of an fp32 value to the 8-bit-mantissa bf16 format. */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) /* NaN stays NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16, lower = u & 0xFFFFu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

void oracle_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(in[i]);
}

/* ---------------------------------------------------------------- row-parallel helper */
typedef void (*row_fn)(void* ctx, int64_t r0, int64_t r1);
typedef struct { row_fn fn; void* ctx; int64_t r0, r1; } row_job;

static void* row_job_run(void* p) {
    row_job* j = (row_job*)p;
    if (j->r1 > j->r0) j->fn(j->ctx, j->r0, j->r1);
    return NULL;
}

/* Static partition of rows [0, rows) over the oracle's threads. */
static void parallel_rows(int64_t rows, row_fn fn, void* ctx) {
    int nt = oracle_threads();
    if (nt > rows) nt = (int)(rows > 0 ? rows : 1);
    if (nt <= 1) { fn(ctx, 0, rows); return; }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    row_job* jobs = (row_job*)malloc(sizeof(row_job) * (size_t)nt);
    for (int t = 0; t < nt; ++t) {
        jobs[t].fn = fn; jobs[t].ctx = ctx;
        jobs[t].r0 = rows * t / nt; jobs[t].r1 = rows * (t + 1) / nt;
        pthread_create(&th[t], NULL, row_job_run, &jobs[t]);
    }
    for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
    free(th); free(jobs);
}

/* ---------------------------------------------------------------- O1: calibration max-abs */
/* s_j = max over rows m of |X_mj|  ([PTQ] W8A8 recipe: per-channel activation scale s). */
void oracle_channel_absmax(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, float* s, int accumulate) {
    if (!accumulate)
        for (int64_t j = 0; j < K; ++j) s[j] = 0.0f;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < K; ++j) {
            float v = fabsf(oracle_bf16_to_f32(X[m * ldx + j]));
            if (v > s[j]) s[j] = v;
        }
}

/* ---------------------------------------------------------------- O2: smoothing vector */
/* lambda_j = s_j^alpha / w_j^(1-alpha) with w_j = max_i |W_ij|  ([PTQ] W8A8 recipe). */
void oracle_smooth_lambda(const float* s, const float* w, int64_t K, float alpha, float* lambda,
                          float* inv_lambda) {
    for (int64_t j = 0; j < K; ++j) {
        float l;
        if (s[j] == 0.0f || w[j] == 0.0f)
            l = 1.0f;
        else if (alpha == 0.5f)
            l = sqrtf(s[j]) / sqrtf(w[j]);
        else
            l = powf(s[j], alpha) / powf(w[j], 1.0f - alpha);
        lambda[j] = l;
        inv_lambda[j] = 1.0f / l;
    }
}

/* ---------------------------------------------------------------- O3/O4: per-row INT8 */
typedef struct {
    const uint16_t* X; const float* colmul; int64_t K, ldx; int8_t* q; float* scale;
} quant_ctx;

static void quant_rows(void* p, int64_t r0, int64_t r1) {
    quant_ctx* c = (quant_ctx*)p;
    float* v = (float*)malloc(sizeof(float) * (size_t)c->K);
    for (int64_t m = r0; m < r1; ++m) {
        const uint16_t* x = c->X + m * c->ldx;
        float amax = 0.0f;
        for (int64_t j = 0; j < c->K; ++j) {
            float f = oracle_bf16_to_f32(x[j]);
            v[j] = c->colmul ? f * c->colmul[j] : f;
            float a = fabsf(v[j]);
            if (a > amax) amax = a;
        }
        int8_t* q = c->q + m * c->K;
        if (amax == 0.0f) {
            c->scale[m] = 0.0f;
            for (int64_t j = 0; j < c->K; ++j) q[j] = 0;
            continue;
        }
        float sc = amax / 127.0f;
        c->scale[m] = sc;
        for (int64_t j = 0; j < c->K; ++j) {
            float t = rintf(v[j] / sc); /* default rounding mode: half to even */
            if (t > 127.0f) t = 127.0f;
            if (t < -127.0f) t = -127.0f;
            q[j] = (int8_t)t;
        }
    }
    free(v);
}

/* Row m: v = X_m * colmul (elementwise, colmul may be NULL), scale_m = max|v| / 127,
 * q = clamp(rint(v / scale_m), -127, 127).  Used with colmul = inv_lambda for the
 * activations (per token) and colmul = lambda for the weights (per output row). */
void oracle_quantize_rows(const uint16_t* X, const float* colmul, int64_t M, int64_t K, int64_t ldx,
                          int8_t* q, float* scale) {
    quant_ctx c = {X, colmul, K, ldx, q, scale};
    parallel_rows(M, quant_rows, &c);
}

/* Offline weight preparation: w_j, lambda, inv_lambda, then Wq/sw from W * diag(lambda).
 * s == NULL means no smoothing (lambda = 1). */
void oracle_smooth_prepare(const uint16_t* W, const float* s, int64_t N, int64_t K, float alpha,
                           int8_t* Wq, float* sw, float* inv_lambda, float* lambda) {
    float* w = (float*)malloc(sizeof(float) * (size_t)K);
    float* lam = lambda ? lambda : (float*)malloc(sizeof(float) * (size_t)K);
    float* inv = inv_lambda ? inv_lambda : (float*)malloc(sizeof(float) * (size_t)K);
    if (s) {
        oracle_channel_absmax(W, N, K, K, w, 0);
        oracle_smooth_lambda(s, w, K, alpha, lam, inv);
    } else {
        for (int64_t j = 0; j < K; ++j) { lam[j] = 1.0f; inv[j] = 1.0f; }
    }
    oracle_quantize_rows(W, s ? lam : NULL, N, K, K, Wq, sw);
    free(w);
    if (!lambda) free(lam);
    if (!inv_lambda) free(inv);
}

/* ---------------------------------------------------------------- O5: integer GEMM */
typedef struct {
    const int8_t* A; const int8_t* B; int64_t N, K; int32_t* C32; int64_t* C64;
} gemm_ctx;

static void gemm_rows(void* p, int64_t r0, int64_t r1) {
    gemm_ctx* c = (gemm_ctx*)p;
    for (int64_t m = r0; m < r1; ++m) {
        const int8_t* a = c->A + m * c->K;
        for (int64_t n = 0; n < c->N; ++n) {
            const int8_t* b = c->B + n * c->K;
            if (c->C32) {
                uint32_t acc = 0; /* int32 two's-complement accumulation without UB */
                for (int64_t k = 0; k < c->K; ++k) acc += (uint32_t)((int32_t)a[k] * (int32_t)b[k]);
                c->C32[m * c->N + n] = (int32_t)acc;
            } else {
                int64_t acc = 0;
                for (int64_t k = 0; k < c->K; ++k) acc += (int64_t)a[k] * (int64_t)b[k];
                c->C64[m * c->N + n] = acc;
            }
        }
    }
}

/* C[m][n] = sum_k A[m][k] * B[n][k]: activations [M,K] times weights [N,K] transposed. */
void oracle_gemm_i32(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t K, int32_t* C) {
    gemm_ctx c = {A, B, N, K, C, NULL};
    parallel_rows(M, gemm_rows, &c);
}

void oracle_gemm_i64(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t K, int64_t* C) {
    gemm_ctx c = {A, B, N, K, NULL, C};
    parallel_rows(M, gemm_rows, &c);
}

/* ---------------------------------------------------------------- O6: epilogues */
static float dequant_bias(int32_t acc, float sx, float sw, const uint16_t* bias, int64_t n) {
    float b = bias ? oracle_bf16_to_f32(bias[n]) : 0.0f;
    float d = sx * sw;
    return fmaf((float)acc, d, b);
}

/* One output row.  acc: [N] (N = 2F for SILU_GATE), Y: [N_out]. */
static void epilogue_row(const int32_t* acc, int64_t N, float sx, const float* sw, const uint16_t* bias,
                         int epi, const uint16_t* gamma, int64_t head_dim, float eps, uint16_t* Y,
                         float* ybuf) {
    if (epi == ORACLE_EPI_BIAS) {
        for (int64_t n = 0; n < N; ++n) Y[n] = oracle_f32_to_bf16(dequant_bias(acc[n], sx, sw[n], bias, n));
    } else if (epi == ORACLE_EPI_SILU_GATE) {
        int64_t F = N / 2;
        for (int64_t f = 0; f < F; ++f) {
            float g = dequant_bias(acc[f], sx, sw[f], bias, f);
            float u = dequant_bias(acc[F + f], sx, sw[F + f], bias, F + f);
            float silu = g / (1.0f + expf(-g));
            Y[f] = oracle_f32_to_bf16(silu * u);
        }
    } else { /* ORACLE_EPI_HEAD_RMSNORM */
        for (int64_t n = 0; n < N; ++n) ybuf[n] = dequant_bias(acc[n], sx, sw[n], bias, n);
        for (int64_t h0 = 0; h0 < N; h0 += head_dim) {
            double ss = 0.0;
            for (int64_t d = 0; d < head_dim; ++d) ss += (double)ybuf[h0 + d] * (double)ybuf[h0 + d];
            float ms = (float)ss / (float)head_dim;
            float r = 1.0f / sqrtf(ms + eps);
            for (int64_t d = 0; d < head_dim; ++d) {
                float g = oracle_bf16_to_f32(gamma[d]);
                Y[h0 + d] = oracle_f32_to_bf16((ybuf[h0 + d] * r) * g);
            }
        }
    }
}

typedef struct {
    const int32_t* acc; int64_t N; const float* sx; const float* sw; const uint16_t* bias; int epi;
    const uint16_t* gamma; int64_t head_dim; float eps; uint16_t* Y; int64_t ldy;
} epi_ctx;

static void epi_rows(void* p, int64_t r0, int64_t r1) {
    epi_ctx* c = (epi_ctx*)p;
    float* ybuf = (float*)malloc(sizeof(float) * (size_t)c->N);
    for (int64_t m = r0; m < r1; ++m)
        epilogue_row(c->acc + m * c->N, c->N, c->sx[m], c->sw, c->bias, c->epi, c->gamma, c->head_dim, c->eps,
                     c->Y + m * c->ldy, ybuf);
    free(ybuf);
}

/* Y[m][:] = epilogue(acc[m][:]) for all M rows; acc is [M, N] int32 row-major. */
void oracle_epilogue(const int32_t* acc, int64_t M, int64_t N, const float* sx, const float* sw,
                     const uint16_t* bias, int epi, const uint16_t* gamma, int64_t head_dim, float eps,
                     uint16_t* Y, int64_t ldy) {
    epi_ctx c = {acc, N, sx, sw, bias, epi, gamma, head_dim, eps, Y, ldy};
    parallel_rows(M, epi_rows, &c);
}

/* ---------------------------------------------------------------- sampled rows */
typedef struct {
    const int8_t* Xq; const float* sx; const int8_t* Wq; const float* sw; const uint16_t* bias;
    const int64_t* rows; int64_t N, K; int epi; const uint16_t* gamma; int64_t head_dim; float eps;
    uint16_t* Y; int64_t ldy; int32_t* acc_out;
} rows_ctx;

static void linear_rows_run(void* p, int64_t i0, int64_t i1) {
    rows_ctx* c = (rows_ctx*)p;
    int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * (size_t)c->N);
    float* ybuf = (float*)malloc(sizeof(float) * (size_t)c->N);
    for (int64_t i = i0; i < i1; ++i) {
        int64_t m = c->rows[i];
        gemm_ctx g = {c->Xq + m * c->K, c->Wq, c->N, c->K, acc, NULL};
        gemm_rows(&g, 0, 1);
        if (c->acc_out) memcpy(c->acc_out + i * c->N, acc, sizeof(int32_t) * (size_t)c->N);
        if (c->Y)
            epilogue_row(acc, c->N, c->sx[m], c->sw, c->bias, c->epi, c->gamma, c->head_dim, c->eps,
                         c->Y + i * c->ldy, ybuf);
    }
    free(acc); free(ybuf);
}

/* GEMM + epilogue for the listed rows only (rows are independent): output row i of
 * Y / acc_out belongs to input row rows[i].  Y or acc_out may be NULL. */
void oracle_linear_rows(const int8_t* Xq, const float* sx, const int8_t* Wq, const float* sw,
                        const uint16_t* bias, const int64_t* rows, int64_t nrows, int64_t N, int64_t K, int epi,
                        const uint16_t* gamma, int64_t head_dim, float eps, uint16_t* Y, int64_t ldy,
                        int32_t* acc_out) {
    rows_ctx c = {Xq, sx, Wq, sw, bias, rows, N, K, epi, gamma, head_dim, eps, Y, ldy, acc_out};
    parallel_rows(nrows, linear_rows_run, &c);
}

/* ---------------------------------------------------------------- O7: bf16 GEMM */
typedef struct {
    const uint16_t* H; const uint16_t* W; const uint16_t* bias; const int64_t* rows; int64_t N, K;
    uint16_t* Z; float* Zf;
} bgemm_ctx;

static void bgemm_rows(void* p, int64_t i0, int64_t i1) {
    bgemm_ctx* c = (bgemm_ctx*)p;
    for (int64_t i = i0; i < i1; ++i) {
        int64_t m = c->rows ? c->rows[i] : i;
        const uint16_t* h = c->H + m * c->K;
        for (int64_t n = 0; n < c->N; ++n) {
            const uint16_t* w = c->W + n * c->K;
            double acc = 0.0; /* bf16 x bf16 products are exact in fp64 */
            for (int64_t k = 0; k < c->K; ++k)
                acc += (double)oracle_bf16_to_f32(h[k]) * (double)oracle_bf16_to_f32(w[k]);
            if (c->bias) acc += (double)oracle_bf16_to_f32(c->bias[n]);
            float f = (float)acc;
            if (c->Zf) c->Zf[i * c->N + n] = f;
            c->Z[i * c->N + n] = oracle_f32_to_bf16(f);
        }
    }
}

/* Z = H * W^T (+ bias): H [M,K], W [N,K] bf16; Z [nrows, N] bf16 and optional fp32 Zf.
 * rows == NULL computes every row (nrows = M). */
void oracle_bf16_gemm_rows(const uint16_t* H, const uint16_t* W, const uint16_t* bias, const int64_t* rows,
                           int64_t nrows, int64_t N, int64_t K, uint16_t* Z, float* Zf) {
    bgemm_ctx c = {H, W, bias, rows, N, K, Z, Zf};
    parallel_rows(nrows, bgemm_rows, &c);
}

/* ---------------------------------------------------------------- O8: adaLN modulation */
typedef struct {
    const uint16_t* X; int64_t ldx; const uint16_t* shift; const uint16_t* scale; float eps; int64_t K;
    uint16_t* H;
} adaln_ctx;

static void adaln_rows(void* p, int64_t r0, int64_t r1) {
    adaln_ctx* c = (adaln_ctx*)p;
    for (int64_t m = r0; m < r1; ++m) {
        const uint16_t* x = c->X + m * c->ldx;
        double sum = 0.0;
        for (int64_t j = 0; j < c->K; ++j) sum += (double)oracle_bf16_to_f32(x[j]);
        double mean = sum / (double)c->K;
        double ss = 0.0;
        for (int64_t j = 0; j < c->K; ++j) {
            double d = (double)oracle_bf16_to_f32(x[j]) - mean;
            ss += d * d;
        }
        float mu = (float)mean;
        float var = (float)(ss / (double)c->K);
        float r = 1.0f / sqrtf(var + c->eps);
        uint16_t* h = c->H + m * c->K;
        for (int64_t j = 0; j < c->K; ++j) {
            float n = (oracle_bf16_to_f32(x[j]) - mu) * r;
            float g = 1.0f + (c->scale ? oracle_bf16_to_f32(c->scale[j]) : 0.0f);
            float b = c->shift ? oracle_bf16_to_f32(c->shift[j]) : 0.0f;
            h[j] = oracle_f32_to_bf16(n * g + b);
        }
    }
}

/* H = bf16(LayerNorm(X) * (1 + scale) + shift) per row; shift / scale [K] bf16 or NULL (0).
 * H is [M, K] row-major.  The activations for the next linear are quantize_rows(H, inv_lambda). */
void oracle_adaln_modulate(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, const uint16_t* shift,
                           const uint16_t* scale, float eps, uint16_t* H) {
    adaln_ctx c = {X, ldx, shift, scale, eps, K, H};
    parallel_rows(M, adaln_rows, &c);
}

/* ---------------------------------------------------------------- O9: MXFP4 (block-scaled FP4) */
/* Magnitudes of the eight 4-bit codes 0..7: exponent field e (2 bits, bias 1) and mantissa m
 * (1 bit): e = 0 gives m * 0.5, e > 0 gives (1 + m / 2) * 2^(e - 1). */
double oracle_fp4_value(int code) {
    int idx = code & 7, e = idx >> 1, m = idx & 1;
    double mag = e == 0 ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
    return (code & 8) ? -mag : mag;
}

/* Nearest of the eight magnitudes to |t|, ties to the code with mantissa bit 0; saturates. */
static int fp4_round_index(double a) {
    int best = 0;
    double bd = INFINITY;
    for (int i = 0; i < 8; ++i) {
        double d = fabs(a - oracle_fp4_value(i));
        if (d < bd || (d == bd && (i & 1) == 0)) { bd = d; best = i; }
    }
    return best;
}

typedef struct {
    const uint16_t* X; const float* colmul; int64_t K, ldx; uint8_t* q; uint8_t* s;
} mx_ctx;

static void mx_rows(void* p, int64_t r0, int64_t r1) {
    mx_ctx* c = (mx_ctx*)p;
    for (int64_t m = r0; m < r1; ++m) {
        const uint16_t* x = c->X + m * c->ldx;
        for (int64_t b = 0; b < c->K / 32; ++b) {
            float v[32];
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                int64_t j = b * 32 + i;
                float f = oracle_bf16_to_f32(x[j]);
                v[i] = c->colmul ? f * c->colmul[j] : f;
                if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
            }
            int e = -127;
            if (amax > 0.0f) {
                int ex;
                frexpf(amax, &ex);         /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
                e = (ex - 1) - 2;
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            c->s[m * (c->K / 32) + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; ++i) {
                double t = ldexp((double)v[i], -e);  /* exact: a power-of-two scaling in fp64 */
                int idx = fp4_round_index(fabs(t));
                int code = idx == 0 ? 0 : ((t < 0.0 ? 8 : 0) | idx);
                int64_t j = b * 32 + i;
                uint8_t* qb = c->q + m * (c->K / 2) + j / 2;
                if (j % 2 == 0) *qb = (uint8_t)code; else *qb = (uint8_t)(*qb | (code << 4));
            }
        }
    }
}

/* Row m of X (times colmul when given): codes Q [M, K/2] and biased block exponents S [M, K/32]. */
void oracle_mxfp4_quantize_rows(const uint16_t* X, const float* colmul, int64_t M, int64_t K, int64_t ldx,
                                uint8_t* Q, uint8_t* S) {
    mx_ctx c = {X, colmul, K, ldx, Q, S};
    parallel_rows(M, mx_rows, &c);
}

/* Element j of a quantized row: code value times its block's power of two. */
static double mx_elem(const uint8_t* q, const uint8_t* s, int64_t j) {
    int code = (j % 2 == 0) ? (q[j / 2] & 15) : (q[j / 2] >> 4);
    return ldexp(oracle_fp4_value(code), (int)s[j / 32] - 127);
}

typedef struct {
    const uint8_t* Xq; const uint8_t* Xs; const uint8_t* Wq; const uint8_t* Ws; const uint16_t* bias;
    const int64_t* rows; int64_t N, K; int epi; const uint16_t* gamma; float eps; double* acc; uint16_t* Y;
} mxg_ctx;

static void mxg_rows(void* p, int64_t i0, int64_t i1) {
    mxg_ctx* c = (mxg_ctx*)p;
    double* a = (double*)malloc(sizeof(double) * (size_t)c->N);
    for (int64_t i = i0; i < i1; ++i) {
        int64_t m = c->rows ? c->rows[i] : i;
        const uint8_t* xq = c->Xq + m * (c->K / 2);
        const uint8_t* xs = c->Xs + m * (c->K / 32);
        for (int64_t n = 0; n < c->N; ++n) {
            const uint8_t* wq = c->Wq + n * (c->K / 2);
            const uint8_t* ws = c->Ws + n * (c->K / 32);
            double s = 0.0; /* products are exact; the fp64 sum rounds far below fp32 */
            for (int64_t k = 0; k < c->K; ++k) s += mx_elem(xq, xs, k) * mx_elem(wq, ws, k);
            a[n] = s;
            if (c->acc) c->acc[i * c->N + n] = s;
        }
        if (!c->Y) continue;
        if (c->epi == ORACLE_EPI_SILU_GATE) {
            int64_t F = c->N / 2;
            for (int64_t f = 0; f < F; ++f) {
                float g = (float)a[f] + (c->bias ? oracle_bf16_to_f32(c->bias[f]) : 0.0f);
                float u = (float)a[F + f] + (c->bias ? oracle_bf16_to_f32(c->bias[F + f]) : 0.0f);
                c->Y[i * F + f] = oracle_f32_to_bf16((g / (1.0f + expf(-g))) * u);
            }
        } else if (c->epi == ORACLE_EPI_HEAD_RMSNORM) {
            for (int64_t h0 = 0; h0 < c->N; h0 += 256) {
                float y[256];
                double ss = 0.0;
                for (int d = 0; d < 256; ++d) {
                    y[d] = (float)a[h0 + d] + (c->bias ? oracle_bf16_to_f32(c->bias[h0 + d]) : 0.0f);
                    ss += (double)y[d] * (double)y[d];
                }
                float ms = (float)ss / 256.0f;
                float r = 1.0f / sqrtf(ms + c->eps);
                for (int d = 0; d < 256; ++d)
                    c->Y[i * c->N + h0 + d] = oracle_f32_to_bf16((y[d] * r) * oracle_bf16_to_f32(c->gamma[d]));
            }
        } else {
            for (int64_t n = 0; n < c->N; ++n) {
                float b = c->bias ? oracle_bf16_to_f32(c->bias[n]) : 0.0f;
                c->Y[i * c->N + n] = oracle_f32_to_bf16((float)a[n] + b);
            }
        }
    }
    free(a);
}

/* acc[i][n] = sum_k dec(X row rows[i], k) * dec(W row n, k) (fp64), then with y = (float)acc + bias
 * (fp32): BIAS Y = bf16(y); SILU_GATE (W rows [gate; up], N = 2F) Y[i][f] = bf16((g / (1 + expf(-g)))
 * * u) with g, u the gate and up values of y; HEAD_RMSNORM per 256-column head as the W8A8 epilogue
 * (fp64 sum of y^2, r = 1 / sqrtf(ms + eps), Y = bf16((y * r) * gamma)).
 * rows == NULL computes every row; acc or Y may be NULL. */
void oracle_mxfp4_gemm_rows(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                            const uint16_t* bias, const int64_t* rows, int64_t nrows, int64_t N, int64_t K, int epi,
                            const uint16_t* gamma, float eps, double* acc, uint16_t* Y) {
    mxg_ctx c = {Xq, Xs, Wq, Ws, bias, rows, N, K, epi, gamma, eps, acc, Y};
    parallel_rows(nrows, mxg_rows, &c);
}

/* ---------------------------------------------------------------- O11: weight-only blocks */
/* fp32 -> IEEE binary16 bits, round half to even, subnormal halves kept; magnitudes that would
 * round to infinity (from 65520 up) saturate to the largest finite half, 65504.  Finite input. */
uint16_t oracle_f32_to_f16(float f) {
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (a >= 65520.0) return sign | 0x7BFF;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: units of 2^-24 (1024 units = 2^-14 is the smallest normal, whose
         * encoding 0x0400 continues the same count) */
        double units = nearbyint(a * ldexp(1.0, 24));
        return sign | (uint16_t)units;
    }
    int e2;
    frexp(a, &e2);               /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;              /* a in [2^e, 2^(e+1)) */
    double m = nearbyint(ldexp(a, 10 - e));  /* 11-bit significand in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; e += 1; }
    return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

/* IEEE binary16 bits -> value (exact in fp32 and fp64). */
double oracle_f16_to_f64(uint16_t h) {
    int e = (h >> 10) & 31, m = h & 1023;
    double v = e == 0 ? ldexp((double)m, -24) : ldexp((double)(1024 + m), e - 25);
    return (h & 0x8000) ? -v : v;
}

typedef struct {
    const uint16_t* W; int64_t K, ldw; int bits; uint8_t* Q; uint16_t* D;
} wo_ctx;

static void wo_rows(void* p, int64_t r0, int64_t r1) {
    wo_ctx* c = (wo_ctx*)p;
    const int qmax = c->bits == 8 ? 127 : 7;
    for (int64_t n = r0; n < r1; ++n) {
        const uint16_t* w = c->W + n * c->ldw;
        for (int64_t b = 0; b < c->K / 32; ++b) {
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j) {
                float v = fabsf(oracle_bf16_to_f32(w[b * 32 + j]));
                if (v > amax) amax = v;
            }
            uint16_t dh = oracle_f32_to_f16(amax / (float)qmax);
            float d = (float)oracle_f16_to_f64(dh);
            c->D[n * (c->K / 32) + b] = dh;
            for (int j = 0; j < 32; ++j) {
                int64_t k = b * 32 + j;
                int q = 0;
                if (d > 0.0f) {
                    float t = rintf(oracle_bf16_to_f32(w[k]) / d);
                    if (t > (float)qmax) t = (float)qmax;
                    if (t < (float)-qmax) t = (float)-qmax;
                    q = (int)t;
                }
                if (c->bits == 8) {
                    c->Q[n * c->K + k] = (uint8_t)(int8_t)q;
                } else {
                    uint8_t* byte = &c->Q[n * (c->K / 2) + k / 2];
                    *byte = (k % 2 == 0) ? (uint8_t)((*byte & 0xF0) | (q + 8)) : (uint8_t)((*byte & 0x0F) | ((q + 8) << 4));
                }
            }
        }
    }
}

/* Weight-only quantization of W [N, ldw] (first K columns, K % 32 == 0): codes Q ([N, K] int8
 * for bits = 8, [N, K/2] nibbles for bits = 4) and half scales D [N, K/32]. */
void oracle_wo_quantize(const uint16_t* W, int64_t N, int64_t K, int64_t ldw, int bits, uint8_t* Q, uint16_t* D) {
    wo_ctx c = {W, K, ldw, bits, Q, D};
    parallel_rows(N, wo_rows, &c);
}

/* Signed code of element k of a quantized row. */
static int wo_code(const uint8_t* q, int64_t k, int bits) {
    if (bits == 8) return (int)(int8_t)q[k];
    int nib = (k % 2 == 0) ? (q[k / 2] & 15) : (q[k / 2] >> 4);
    return nib - 8;
}

/* Dequantized weights Wd [N, K] bf16: Wd[n][k] = bf16(q * d) (the product is exact). */
void oracle_wo_dequantize(const uint8_t* Q, const uint16_t* D, int64_t N, int64_t K, int bits, uint16_t* Wd) {
    const int64_t qrow = bits == 8 ? K : K / 2;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            double v = (double)wo_code(Q + n * qrow, k, bits) * oracle_f16_to_f64(D[n * (K / 32) + k / 32]);
            Wd[n * K + k] = oracle_f32_to_bf16((float)v);
        }
}

/* ---------------------------------------------------------------- O12: attention */
typedef struct {
    const uint16_t* Q; const uint16_t* K; const uint16_t* V; int64_t S, ld; const int64_t* rows; int64_t h;
    uint16_t* O; double* acc;
} attn_ctx;

static void attn_rows(void* p, int64_t i0, int64_t i1) {
    attn_ctx* c = (attn_ctx*)p;
    double* sc = (double*)malloc(sizeof(double) * (size_t)c->S);
    double o[256];
    for (int64_t i = i0; i < i1; ++i) {
        int64_t m = c->rows ? c->rows[i] : i;
        const uint16_t* q = c->Q + m * c->ld + c->h * 256;
        double mx = -INFINITY;
        for (int64_t j = 0; j < c->S; ++j) {
            const uint16_t* k = c->K + j * c->ld + c->h * 256;
            double d = 0.0; /* bf16 x bf16 products are exact in fp64 */
            for (int t = 0; t < 256; ++t) d += (double)oracle_bf16_to_f32(q[t]) * (double)oracle_bf16_to_f32(k[t]);
            sc[j] = d / 16.0;
            if (sc[j] > mx) mx = sc[j];
        }
        double l = 0.0;
        for (int t = 0; t < 256; ++t) o[t] = 0.0;
        for (int64_t j = 0; j < c->S; ++j) {
            double pj = exp(sc[j] - mx);
            const uint16_t* v = c->V + j * c->ld + c->h * 256;
            l += pj;
            for (int t = 0; t < 256; ++t) o[t] += pj * (double)oracle_bf16_to_f32(v[t]);
        }
        for (int t = 0; t < 256; ++t) {
            double y = o[t] / l;
            if (c->acc) c->acc[i * 256 + t] = y;
            c->O[i * 256 + t] = oracle_f32_to_bf16((float)y);
        }
    }
    free(sc);
}

/* Head h of the attention for the listed query rows (rows == NULL: rows 0 .. nrows - 1): output
 * row i (bf16 [nrows, 256], and the fp64 values when acc is not NULL) belongs to query rows[i]. */
void oracle_attention_rows(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t S, int64_t ld, int64_t h,
                           const int64_t* rows, int64_t nrows, uint16_t* O, double* acc) {
    attn_ctx c = {Q, K, V, S, ld, rows, h, O, acc};
    parallel_rows(nrows, attn_rows, &c);
}
