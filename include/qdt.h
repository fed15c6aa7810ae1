/*
 * qdt.h -- C ABI of the W8A8 quantized linear of a flow-matching diffusion transformer,
 * implemented in hand-written HIP for AMD CDNA4 (gfx950, MI355X).
 *
 * The layer (pages, by title):
 *   [PTQ]  "Quantizing a Dual-Branch Flow-Matching Diffusion Transformer for Consumer GPUs:
 *          INT8 and GGUF Post-Training Quantization of Ideogram 4.0", W8A8 recipe paragraph:
 *          per-output-row INT8 weights, per-token dynamic INT8 activations, SmoothQuant
 *          smoothing lambda_j = s_j^alpha / max_i |W_ij|^(1-alpha) with alpha = 0.5 that
 *          scales activations down and weights up before quantization; the FFN
 *          down-projections are kept in bf16 (fragility paragraph).
 *   [FAL]  "Serving sub-second Ideogram v4 without quality loss", paragraph on fused
 *          epilogues: the small op after each big matmul (RMSNorm over 256-wide heads,
 *          gated SiLU) is fused into the GEMM.
 *   [ZC]   "Faster Ideogram 4 with Less Prompt Compute", section "Most of the Tensor Was
 *          Zero": a linear with bias, rows projected independently, zero rows give the bias.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers into memory of the current HIP device; the caller
 *     owns every buffer.  The library allocates no device memory.
 *   - bf16 tensors are passed as uint16_t bit patterns.  Matrices are row-major; W is
 *     [out_features = N, in_features = K] (nn.Linear layout), X is [M tokens, K].
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call
 *     enqueues its kernels on `stream` and returns without synchronizing.
 *   - Errors: argument errors are detected on the host before anything is launched and
 *     returned synchronously (nothing is enqueued then).  A launch failure returns
 *     QDT_EHIP.  Faults inside a kernel surface at the caller's next synchronization.
 *   - Alignment: every pointer 16-byte aligned; row strides (ld*) in elements with
 *     (ld * element size) a multiple of 16 bytes.
 *   - K must be a positive multiple of 64 (of 128 for qdt_w8a8_linear, whose main loop
 *     moves whole 128-byte cache lines per row and stage) and at most QDT_MAX_K (the int32
 *     accumulator bound 127^2 * K < 2^31 holds up to K = 133144).
 *   - Floating point follows IEEE fp32 round-to-nearest-even with no contraction except
 *     the explicit fused multiply-add named below; integer stages are exact.
 */
#ifndef QDT_H
#define QDT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QDT_MAX_K 131072

typedef enum qdt_status {
    QDT_OK = 0,
    QDT_EINVAL = 1,       /* null pointer, bad enum or parameter value */
    QDT_ESHAPE = 2,       /* dimension not supported (K % 64 or % 128, N % 16, head_dim, ...) */
    QDT_EALIGN = 3,       /* pointer or row stride misaligned */
    QDT_EWORKSPACE = 4,   /* workspace missing or smaller than required */
    QDT_EALIAS = 5,       /* output overlaps an input */
    QDT_EHIP = 6,         /* the HIP runtime reported an error at launch */
    QDT_EUNSUPPORTED = 7  /* valid request the library does not implement (e.g. plan/epilogue pair) */
} qdt_status;

typedef enum qdt_epilogue {
    /* Y[m][n] = bf16_rne(fmaf((float)acc[m][n], x_scale[m] * w_scale[n], bias[n]))
     * (bias term +0.0f when bias is NULL).  [PTQ] dequantization; [ZC] linear with bias. */
    QDT_EPI_BIAS = 0,
    /* W rows are [gate(0..F-1); up(F..2F-1)], N = 2F, Y is [M, F]:
     * g, u as in BIAS on rows f and F+f; Y[m][f] = bf16_rne((g / (1 + expf(-g))) * u).
     * [FAL] gated-SiLU epilogue. */
    QDT_EPI_SILU_GATE = 1,
    /* y as in BIAS; per row and per head of head_dim columns: r = 1/sqrtf(mean(y^2) + eps),
     * Y = bf16_rne((y * r) * gamma[n mod head_dim]).  [FAL] RMSNorm over 256-wide heads. */
    QDT_EPI_HEAD_RMSNORM = 2,
    /* Y is int32 [M, N]: the raw accumulators sum_k Xq[m][k] * Wq[n][k] (for testing). */
    QDT_EPI_ACC_I32 = 3,
    /* Y is fp32 [M, N]: the raw accumulators of qdt_mxfp4_linear or qdt_wo_linear (for testing). */
    QDT_EPI_ACC_F32 = 4
} qdt_epilogue;

/* Parameters of QDT_EPI_HEAD_RMSNORM.  gamma: device bf16 [head_dim], shared by all heads. */
typedef struct qdt_rmsnorm_params {
    const uint16_t* gamma;
    int32_t head_dim; /* must be 256 */
    float eps;        /* added to the mean square inside the square root */
} qdt_rmsnorm_params;

/* Workgroup tile shapes of the MFMA GEMM. */
typedef enum qdt_tile {
    QDT_TILE_AUTO = -1,
    QDT_TILE_256 = 0,    /* 256 token rows x 256 weight rows per workgroup */
    QDT_TILE_288 = 1,    /* 288 x 288: 16 x 16 = 256 tiles at 4608 x 4608, one per compute unit */
    QDT_TILE_288x256 = 2, /* 288 token rows x 256 weight rows (any epilogue); only on request: the
                             planner does not pick it (slower per tile than 256 x 256 on the FFN) */
    QDT_TILE_224x256 = 3  /* 224 token rows x 256 weight rows (any epilogue): more, smaller tiles where
                             256-row tiles leave a last round of workgroups mostly empty (6037 tokens:
                             486 tiles in two full rounds instead of 432 in 1.69) */
} qdt_tile;

/* Launch plan of qdt_w8a8_linear.  The planner fills every field; callers of
 * qdt_w8a8_linear_planned set `tile` and `split_k` (others are recomputed). */
typedef struct qdt_linear_plan {
    int32_t tile;            /* qdt_tile */
    int32_t split_k;         /* number of K slices; 1 = no split (epilogue fused in the GEMM) */
    int32_t tile_m, tile_n;  /* token rows and weight rows per workgroup */
    int32_t tiles_m, tiles_n;
    int32_t k_tiles;         /* K stages of the main loop (128 bytes of K each) */
    int32_t grid;            /* workgroups launched by the GEMM kernel */
    int64_t workspace_bytes; /* int32 partial sums for split_k > 1, else 0 */
} qdt_linear_plan;

/* Human-readable name of a status code (static storage). */
const char* qdt_status_string(qdt_status status);

/* Library version string (static storage). */
const char* qdt_version(void);

/*
 * Calibration max-abs: s[j] = max over rows m of |X[m][j]|  ([PTQ]: the per-channel
 * activation scale s of the smoothing rule; here taken from the given activations).
 *   X: bf16 [M, ldx], first K columns used.  s: fp32 [K], output.
 *   accumulate = 0: s is overwritten; accumulate != 0: s = max(s, new) (several batches).
 * Exact (max of exact values).  M = 0 with accumulate = 0 gives s = 0.
 */
qdt_status qdt_channel_absmax(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, float* s,
                              int accumulate, void* stream);

/*
 * Offline weight preparation ([PTQ] W8A8 recipe):
 *   w_j = max_n |W[n][j]|
 *   lambda_j = sqrtf(s_j) / sqrtf(w_j) for alpha = 0.5 (powf(s_j, alpha) / powf(w_j, 1 - alpha)
 *     otherwise); lambda_j = 1 where s_j or w_j is 0;  inv_lambda_j = 1.0f / lambda_j
 *   What_nj = (float)W[n][j] * lambda_j
 *   w_scale[n] = max_j |What_nj| / 127;  Wq[n][j] = clamp(rint(What_nj / w_scale[n]), -127, 127)
 *   (an all-zero row gets w_scale 0 and Wq 0).
 *   W: bf16 [N, K].  s: fp32 [K] calibration max-abs, or NULL for no smoothing (lambda = 1).
 *   Outputs: Wq int8 [N, K], w_scale fp32 [N], inv_lambda fp32 [K], lambda fp32 [K]
 *   (inv_lambda and lambda are always written; the lambda buffer also serves as scratch).
 *   alpha in [0, 1].  Bit-exact with the CPU definition for alpha = 0.5; other alpha use the
 *   device powf.
 */
qdt_status qdt_smooth_prepare(const uint16_t* W, const float* s, int64_t N, int64_t K, float alpha,
                              int8_t* Wq, float* w_scale, float* inv_lambda, float* lambda, void* stream);

/*
 * Per-token dynamic INT8 quantization of the activations ([PTQ] W8A8 recipe):
 *   v = (float)X[m][j] * inv_lambda[j]   (v = (float)X[m][j] when inv_lambda is NULL)
 *   x_scale[m] = max_j |v| / 127;  Xq[m][j] = clamp(rint(v / x_scale[m]), -127, 127)
 *   with a correctly rounded fp32 division and round-half-to-even; an all-zero row gets
 *   x_scale 0 and Xq 0.
 *   X: bf16 [M, ldx] (first K columns).  Xq: int8 [M, K].  x_scale: fp32 [M].
 *   K % 64 == 0 and K <= QDT_MAX_K; ldx >= K, ldx % 8 == 0; pointers 16-byte aligned; no
 *   output may overlap an input or the other output.
 *   Bit-exact.  M = 0 is a no-op.
 */
qdt_status qdt_quantize_per_token(const uint16_t* X, const float* inv_lambda, int64_t M, int64_t K,
                                  int64_t ldx, int8_t* Xq, float* x_scale, void* stream);

/* Largest K of qdt_adaln_quantize (one wavefront holds a row). */
#define QDT_MAX_ADALN_K 8192

/*
 * Producer-fused quantization: the adaptive LayerNorm in front of a quantized linear in a DiT
 * block, and the per-token quantizer of that linear's input, in one pass over each row.  With
 * Xq and x_scale both NULL only H is written (the adaLN alone, for a bf16 consumer).
 * ([PTQ] related work: the adaLN modulation is generated at run time, so it cannot be folded
 * into the weights offline; [FAL] fused-epilogue paragraph: the small op next to a large one is
 * fused so its input never makes a round trip through memory.)  Per row m of X:
 *   mean = sum_j x_j / K;  var = sum_j (x_j - mean)^2 / K   (fp64 sums in any order, rounded to fp32)
 *   r = 1 / sqrtf(var + eps);  n_j = (x_j - mean) * r
 *   h_j = bf16(n_j * (1 + scale_j) + shift_j)               (fp32, no contraction, one rounding)
 *   then x_scale[m] and Xq[m][:] exactly as qdt_quantize_per_token of h with inv_lambda.
 *   X: bf16 [M, ldx] (first K columns), the residual stream.  shift, scale: bf16 [K] modulation
 *   vectors shared by all rows (NULL = 0).  inv_lambda: fp32 [K] of the consumer linear (NULL =
 *   no smoothing).  eps > 0.
 *   Outputs: Xq int8 [M, K], x_scale fp32 [M], and H bf16 [M, K] (the h values) when not NULL.
 *   K % 64 == 0 and K <= QDT_MAX_ADALN_K; ldx >= K, ldx % 8 == 0; pointers 16-byte aligned; no
 *   output may overlap an input or another output.  QDT_EINVAL for eps <= 0 or not finite, for
 *   only one of Xq / x_scale, or for no output at all.
 *   mean and var match the fp64 definition rounded to fp32 except on rare near-ties of that
 *   rounding, where h may differ by 1 bf16 ulp.  Xq and x_scale are bit-exact functions of h.
 *   M = 0 is a no-op.
 */
qdt_status qdt_adaln_quantize(const uint16_t* X, int64_t ldx, const uint16_t* shift, const uint16_t* scale, float eps,
                              const float* inv_lambda, int64_t M, int64_t K, int8_t* Xq, float* x_scale,
                              uint16_t* H, void* stream);

/*
 * Block-scaled FP4 (MXFP4) of the rows of X * colmul, the 4-bit format native to MI355X's matrix
 * cores ([FAL]: the DiT runs in a block-scaled 4-bit floating-point format).  Per block of 32
 * consecutive elements of a row, v = (float)X[m][j] * colmul[j] (v = (float)X[m][j] when colmul is
 * NULL):
 *   e = clamp(floor(log2(max |v|)) - 2, -127, 127)  (-127 for an all-zero block), stored as e + 127
 *   code_j = nearest of {0, 0.5, 1, 1.5, 2, 3, 4, 6} to |v_j| / 2^e (ties to the even mantissa,
 *            saturating at 6), sign in bit 3, zero stored as +0
 *   Q[m][j / 2] holds code_j in its low nibble for even j, high nibble for odd j.
 *   S holds the biased exponents stage-major, uint8 [K/256][M][8]: the 8 blocks of row m in
 *   elements 256 s .. 256 s + 255 sit in the 8 bytes S[s][m][*], block 8 s + w at byte
 *   2 (w % 4) + w / 4 (order w = 0, 4, 1, 5, 2, 6, 3, 7).  A tile of the GEMM then finds a stage's
 *   exponents of its rows in one contiguous span, and a matrix-core lane finds the two blocks it
 *   needs in a stage side by side.
 *   Used for the activations (colmul = inv_lambda or NULL, per step) and for the weights (colmul =
 *   lambda or NULL, offline).  X: bf16 [M, ldx] (first K columns).  Q: uint8 [M, K/2].  S: uint8
 *   M K / 32 bytes as above.  K % 256 == 0, ldx >= K, ldx % 8 == 0; X, colmul and Q 16-byte aligned.
 *   Bit-exact.  M = 0 is a no-op.
 */
qdt_status qdt_mxfp4_quantize(const uint16_t* X, const float* colmul, int64_t M, int64_t K, int64_t ldx,
                              uint8_t* Q, uint8_t* S, void* stream);

/*
 * Block-scaled FP4 linear on the FP4 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4):
 *   acc[m][n] = sum_k dec(Xq, Xs)[m][k] * dec(Wq, Ws)[n][k], dec = code value * 2^(exponent - 127),
 *   accumulated in fp32 (order unspecified: within the fp32 summation bound of the exact sum);
 *   QDT_EPI_BIAS: Y bf16 [M, ldy], Y[m][n] = bf16_rne(acc + (float)bias[n]) (bias NULL = 0);
 *   QDT_EPI_SILU_GATE: W rows [gate(0..F-1); up(F..2F-1)], N = 2F (N % 32 == 0), Y bf16 [M, ldy >= F]:
 *     g = acc[m][f] + bias[f], u = acc[m][F+f] + bias[F+f], Y[m][f] = bf16_rne((g / (1 + exp(-g))) * u)
 *     ([FAL] gated-SiLU epilogue; the exponential and reciprocal as in the W8A8 SILU epilogue);
 *   QDT_EPI_HEAD_RMSNORM: y = acc + bias; per row and head of 256 columns r = 1/sqrtf(mean(y^2) + eps),
 *     Y = bf16_rne((y * r) * gamma[n mod 256]) (epi_params: qdt_rmsnorm_params, as for qdt_w8a8_linear);
 *   QDT_EPI_ACC_F32: Y fp32 [M, ldy], the accumulators.
 *   Xq / Xs: qdt_mxfp4_quantize of the activations ([M, K/2] codes, [K/256][M][8] exponents); Wq /
 *   Ws the same of the weights ([N, K/2], [K/256][N][8]).  K % 256 == 0 (whole 128-byte stages of
 *   codes), N % 16 == 0, ldy >= N (F for the gated SiLU), ldy % 8 == 0; code and Y pointers 16-byte
 *   aligned, exponent pointers 4-byte aligned.  Y must not overlap an input.
 *   When the plan splits K (deep K, few output tiles: qdt_mxfp4_linear_plan), the slices write fp32
 *   partial sums to `workspace` (plan.workspace_bytes = split_k * M * N * 4, 16-byte aligned, caller
 *   owned) and a second kernel adds them in slice order before the epilogue; otherwise workspace may
 *   be NULL.  QDT_EWORKSPACE if it is missing or too small.  M = 0 is a no-op.
 *   The scales of the block exponents are powers of two, so they take no rounding of their own.
 */
qdt_status qdt_mxfp4_linear(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                            const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi,
                            const void* epi_params, void* Y, int64_t ldy, void* workspace, size_t workspace_bytes,
                            void* stream);

/* The plan qdt_mxfp4_linear uses (tile, K split, workspace bytes).  Pure host computation.  FP4
 * takes the tiles QDT_TILE_256, QDT_TILE_288 (not with SILU_GATE or HEAD_RMSNORM) and, on request,
 * QDT_TILE_288x256; the planner chooses as for qdt_w8a8_linear. */
qdt_status qdt_mxfp4_linear_plan(int64_t M, int64_t N, int64_t K, qdt_epilogue epi, qdt_linear_plan* plan);

/* The plan qdt_mxfp4_linear_planned uses for a requested tile (QDT_TILE_AUTO, QDT_TILE_256, _288 or
 * _288x256; QDT_EINVAL for another) and K split (0 = planner's choice).  Pure host computation. */
qdt_status qdt_mxfp4_linear_plan_for(int64_t M, int64_t N, int64_t K, qdt_epilogue epi, int32_t tile,
                                     int32_t split_k, qdt_linear_plan* plan);

/* As qdt_mxfp4_linear with an explicit tile and K split (plan->tile, plan->split_k; the other fields
 * are recomputed and written back).  Without a K split the result does not depend on the tile: every
 * output's K reduction runs through the same MFMA sequence.  A K split changes the fp32 summation
 * order (within the same bound). */
qdt_status qdt_mxfp4_linear_planned(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                                    const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi,
                                    const void* epi_params, void* Y, int64_t ldy, void* workspace,
                                    size_t workspace_bytes, qdt_linear_plan* plan, void* stream);

/*
 * Weight-only block formats ([PTQ] GGUF paragraph: an 8-bit round-to-nearest format at 8.5 bits
 * per weight and a 4-bit one at 4.5 bits per weight; [ZC] "The NF4 Exactness Problem": the text
 * projection is a linear with dequantized 4-bit weights).  Per block of 32 consecutive weights
 * of a row (amax = max |w| of the block, qmax = 127 for bits = 8, 7 for bits = 4):
 *   Wd[n][b] = IEEE half of amax / qmax (round half to even, subnormal halves kept; from 65520 up
 *              saturated to 65504), d its value;
 *   q = clamp(rint(w / d), -qmax, qmax) with a correctly rounded fp32 division, q = 0 when d = 0;
 *   bits = 8: Wq int8 [N, K] holds q;  bits = 4: Wq uint8 [N, K/2] holds q + 8 in a nibble, the
 *   even element in the low nibble.
 * W bf16 [N, ldw] (first K columns, finite), K % 32 == 0, ldw >= K, ldw % 8 == 0; W and Wq
 * 16-byte aligned, Wd 2-byte aligned; no output may overlap an input or the other output.
 * Bit-exact.  N = 0 is a no-op.  Runs once per weight matrix (offline).
 */
#define QDT_WO_KSLICE 8192
qdt_status qdt_wo_quantize(const uint16_t* W, int64_t N, int64_t K, int64_t ldw, int bits, uint8_t* Wq, uint16_t* Wd,
                           void* stream);

/*
 * Weight-only linear on the bf16 matrix cores: with w~[n][k] = bf16_rne(q * d) (q * d is exact),
 *   acc[m][n] = sum_k X[m][k] * w~[n][k], fp32 accumulation of exact products;
 *   QDT_EPI_BIAS: Y bf16 [M, ldy], Y[m][n] = bf16_rne(acc + (float)bias[n]) (bias NULL = 0);
 *   QDT_EPI_ACC_F32: Y fp32 [M, ldy], the accumulators.
 * Batch invariance ([ZC] "The NF4 Exactness Problem": a kernel whose reduction order follows the
 * row count changes the outputs when fewer rows are projected): K is summed in slices of
 * QDT_WO_KSLICE elements by the same instruction sequence for every tile, the slice sums are
 * added in slice order, then the bias.  Y[m][n] depends only on X's row m, the weights of row n,
 * bias[n] and K: it is bit-identical whatever M is, whichever other rows are in the call and
 * wherever row m sits in it.
 *   X bf16 [M, ldx] (first K columns), Wq / Wd from qdt_wo_quantize with the same bits (4 or 8).
 *   K % 512 == 0, N % 16 == 0, ldx >= K, ldx % 8 == 0, ldy >= N, ldy % 8 == 0; X, Wq, bias, Y
 *   16-byte aligned, Wd 2-byte aligned; Y must not overlap an input.
 *   When K > QDT_WO_KSLICE the slices write fp32 partial sums to `workspace`
 *   (qdt_wo_linear_plan: workspace_bytes = split_k * M * N * 4, 16-byte aligned, caller owned, not
 *   overlapping anything else) and a second kernel adds them; otherwise workspace may be NULL.
 *   QDT_EWORKSPACE if it is missing or too small.  M = 0 is a no-op.
 */
qdt_status qdt_wo_linear(const uint16_t* X, int64_t ldx, const uint8_t* Wq, const uint16_t* Wd, int bits,
                         const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi, void* Y,
                         int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/* The plan qdt_wo_linear uses: 256 x 256 tiles, split_k = ceil(K / QDT_WO_KSLICE) for every M.
 * Pure host computation. */
qdt_status qdt_wo_linear_plan(int64_t M, int64_t N, int64_t K, qdt_linear_plan* plan);

/* The plan qdt_w8a8_linear uses for this problem (pure host computation, no device call). */
qdt_status qdt_w8a8_linear_plan(int64_t M, int64_t N, int64_t K, qdt_epilogue epi, qdt_linear_plan* plan);

/* The plan qdt_w8a8_linear_planned uses for a requested tile (qdt_tile, QDT_TILE_AUTO = planner's
 * choice) and K split (0 = planner's choice; a request is rounded down so no slice is empty).
 * Pure host computation. */
qdt_status qdt_w8a8_linear_plan_for(int64_t M, int64_t N, int64_t K, qdt_epilogue epi, int32_t tile, int32_t split_k,
                                    qdt_linear_plan* plan);

/* Bytes of workspace qdt_w8a8_linear needs for this problem (0 when it needs none). */
qdt_status qdt_w8a8_linear_workspace_size(int64_t M, int64_t N, int64_t K, qdt_epilogue epi, size_t* bytes);

/*
 * W8A8 linear: acc[m][n] = sum_k Xq[m][k] * Wq[n][k] in exact int32 on INT8 MFMA, followed by
 * the epilogue `epi` (see qdt_epilogue), all in one kernel unless the plan splits K.
 *   Xq int8 [M, K], x_scale fp32 [M] (from qdt_quantize_per_token); Wq int8 [N, K],
 *   w_scale fp32 [N] (from qdt_smooth_prepare); bias bf16 [N] or NULL.
 *   epi_params: qdt_rmsnorm_params* for QDT_EPI_HEAD_RMSNORM, else ignored (may be NULL).
 *   Y: bf16 [M, ldy] with ldy >= N_out (N_out = N/2 for SILU_GATE, N otherwise), or int32
 *   [M, ldy] for ACC_I32.  Y must not overlap any input.
 *   workspace: device buffer of at least qdt_w8a8_linear_workspace_size() bytes (may be NULL
 *   when that size is 0).
 * Shapes: M >= 0 (rows are masked, any M), K % 128 == 0, N % 16 == 0 (N % 32 == 0 for
 * SILU_GATE, N % 256 == 0 for HEAD_RMSNORM).  K % 128 rather than the MFMA's K step of 64: each
 * main-loop stage copies one whole 128-byte cache line of every operand row into LDS (half-line
 * stages move operands at two thirds of the rate), and the kernel has no masked partial stage;
 * every K of the DiT's linears (4608, 12288, 53248) is a multiple of 128.  Results do not depend on M, the tile or the
 * K split: the integer sum is exact and every output element is computed by the same
 * fp32 operation sequence.
 */
qdt_status qdt_w8a8_linear(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                           const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi,
                           const void* epi_params, void* Y, int64_t ldy, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): qdt_w8a8_linear with the same arguments, results and
 * errors, minus the workspace.  When the plan splits K, the int32 partial sums go to a scratch
 * array the library holds in static device memory, QDT_NOALLOC_SCRATCH_BYTES per device (64 MiB:
 * the 512 x 4608 x 53248 text projection at its 7-way split needs 63 MiB), allocated when the
 * library's code is loaded on a device and held until the process ends.  A plan whose workspace
 * would exceed it returns QDT_EWORKSPACE (qdt_w8a8_linear_workspace_size gives that size); the call
 * itself allocates nothing.  Every slice writes each partial sum it owns before the reduction reads
 * it, so nothing in the scratch needs clearing between calls.  All calls on one device share its
 * scratch: calls that may overlap in time on one device (different streams, threads) race and
 * must be serialized by the caller.
 */
#define QDT_NOALLOC_SCRATCH_BYTES (64ll << 20)
qdt_status qdt_w8a8_linear_noalloc(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                                   const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi,
                                   const void* epi_params, void* Y, int64_t ldy, void* stream);

/* As qdt_w8a8_linear with an explicit tile and K split (plan->tile, plan->split_k; the other
 * fields are recomputed and written back).  Used to show that results are plan-independent. */
qdt_status qdt_w8a8_linear_planned(const int8_t* Xq, const float* x_scale, const int8_t* Wq,
                                   const float* w_scale, const uint16_t* bias, int64_t M, int64_t N,
                                   int64_t K, qdt_epilogue epi, const void* epi_params, void* Y, int64_t ldy,
                                   void* workspace, size_t workspace_bytes, qdt_linear_plan* plan,
                                   void* stream);

/*
 * bf16 linear of a protected (unquantized) layer ([PTQ] fragility paragraph: the FFN
 * down-projections stay in bf16): Y[m][n] = bf16_rne(sum_k X[m][k] * W[n][k] + bias[n]),
 * products exact, accumulated in fp32 on bf16 MFMA (summation order differs from a serial
 * sum; error within the fp32 forward-error bound of a K-term sum).
 *   X bf16 [M, K], W bf16 [N, K], bias bf16 [N] or NULL, Y bf16 [M, ldy].  ldy (>= N, % 8 == 0)
 *   lets the output land in a column window of a wider row-major buffer, as the other linears
 *   allow, e.g. one projection of several written side by side into a shared activation tensor.
 * Shapes: K % 64 == 0, N % 16 == 0, any M >= 0.
 */
qdt_status qdt_bf16_linear(const uint16_t* X, const uint16_t* W, const uint16_t* bias, int64_t M, int64_t N,
                           int64_t K, uint16_t* Y, int64_t ldy, void* stream);

/*
 * Softmax attention per head after the QK-norm projection ([FAL]: 256-wide attention heads over the
 * DiT's joint sequence of text and image tokens).  For every head h and query row m:
 *   s_j = (Q[m] . K[j]) / 16 over the head's 256 columns (1/16 = 1/sqrt(256)), all S keys, no mask;
 *   O[m] = sum_j p_j V[j] / sum_j p_j with p_j = exp(s_j - max_j s_j), rounded to bf16.
 *   Q, K, V, O: bf16 [S, ld] / [S, ldo], head h in columns 256 h .. 256 h + 255 (the layout the
 *   projections write).  Computed with fp32 scores, base-2 exponentials and bf16 probabilities in
 *   the second product, like any bf16 flash-attention kernel, so the result is within a
 *   first-order error bound of the exact one: 2^-9 (bf16 probabilities) plus the fp32 error of the
 *   scores and of the two sums over S keys, times sum_j p_j |V[j]| / sum_j p_j, plus one bf16 ulp.
 *   Each query row is computed independently of the other rows.  The work is 256-query blocks per
 *   head; when the blocks past a whole number of rounds on the 256 compute units would fill at most
 *   half of a last round, each of those blocks is computed as floor(256 / count) key ranges whose
 *   partial outputs, references and row sums are then merged (the same bound; the fp32 summation
 *   order of those blocks' rows differs from a single pass).
 *   ld, ldo >= 256 H, both % 8 == 0; pointers 16-byte aligned; 1 <= H <= 1024, S <= QDT_ATTN_MAX_S.
 *   `workspace`: caller-owned device memory of qdt_attention_workspace_size bytes (past 8192 tokens
 *   V transposed per head, written by a first pass; the waves' rerun flags; the key-range pieces'
 *   partial outputs; 16-byte aligned); no output may overlap an input or the workspace.  Up to 8192
 *   tokens the kernel reads V's rows transposed from LDS instead of a transposed copy (the same
 *   results bit for bit).  S = 0 is a no-op.
 */
#define QDT_ATTN_HEAD_DIM 256
#define QDT_ATTN_MAX_S (1 << 22)
qdt_status qdt_attention(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t S, int64_t H, int64_t ld,
                         uint16_t* O, int64_t ldo, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace qdt_attention needs: H * 256 * roundup(S, 32) * 2 for V transposed when
 * S > 8192 (0 otherwise), plus 16 bytes per workgroup (one int per wave), plus 256 * 258 * 4 bytes
 * per key-range piece when the last round is split (S = 4608, H = 18: 68 blocks x 3 pieces, 53.9 MB).
 * Pure host computation. */
qdt_status qdt_attention_workspace_size(int64_t S, int64_t H, size_t* bytes);

/*
 * Clock record (diagnostic; not part of the layer).  While a buffer is armed, every GEMM kernel
 * that qdt_w8a8_linear, qdt_w8a8_linear_planned, qdt_w8a8_linear_noalloc, qdt_mxfp4_linear and
 * qdt_bf16_linear launch (not their split-K sums) takes the next `grid` entries of it
 * (one per workgroup, in workgroup-id order) as long as they fit; launches that do not fit record
 * nothing.  Entry = 4 uint64: the shader-clock counter (s_memtime) and the 100 MHz real-time
 * counter (s_memrealtime) read by the workgroup's first wave when it starts, then the same two
 * after its last output store is issued.  The shader clock of a launch is therefore
 * sum(cycles) / sum(real ticks) * 100 MHz over its entries.
 *   buf: device memory of `entries` * 32 bytes, 8-byte aligned, owned by the caller, or NULL to
 *   disarm.  Arming resets the fill level.  The setting is process-wide (all devices, all threads);
 *   it adds one uniform branch per kernel when disarmed.  QDT_EINVAL for entries <= 0 with a
 *   buffer, or a misaligned buffer.
 */
qdt_status qdt_clock_record(uint64_t* buf, int64_t entries);

/* Entries of the armed clock record filled so far (pure host computation). */
qdt_status qdt_clock_record_used(int64_t* entries);

#ifdef __cplusplus
}
#endif
#endif /* QDT_H */
