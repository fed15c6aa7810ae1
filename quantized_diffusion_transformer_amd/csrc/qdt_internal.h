// Internal declarations of the HIP path (kernels, launchers, planner).  Not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qdt.h"

namespace qdt {

constexpr int kNumCU = 256;  // MI355X compute units (8 XCDs x 32); the planner sizes grids for it
constexpr int kNumXCD = 8;

// ------------------------------------------------------------------ elementwise / row kernels
hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t st);
hipError_t launch_colmax(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, float* s, hipStream_t st);
hipError_t launch_lambda(const float* s, float* lam_inout, float* inv, int64_t K, float alpha, hipStream_t st);
// Per-row symmetric INT8 of X[m][:K] * colmul (colmul may be null).
hipError_t launch_quant_rows(const uint16_t* X, int64_t ldx, const float* colmul, int64_t M, int64_t K, int8_t* Q,
                             float* scale, hipStream_t st);
// adaLN (LayerNorm, * (1 + scale) + shift, bf16) of X's rows fused with the per-row INT8 of the
// result times colmul; H (bf16 [M, K]) is written when not null.  K <= 8192.
hipError_t launch_adaln_quant(const uint16_t* X, int64_t ldx, const uint16_t* shift, const uint16_t* scale, float eps,
                              const float* colmul, int64_t M, int64_t K, int8_t* Q, float* xscale, uint16_t* H,
                              hipStream_t st);
// Block-scaled FP4 (MXFP4) of X's rows times colmul: codes Q [M, K/2], biased exponents S [M, K/32].
hipError_t launch_mx_quant(const uint16_t* X, int64_t ldx, const float* colmul, int64_t M, int64_t K, uint8_t* Q,
                           uint8_t* S, hipStream_t st);

// ------------------------------------------------------------------ GEMM
// F32BIAS / F32SILU / F32RMSNORM: the fp32-accumulator forms (bf16 and block-scaled FP4 GEMMs) of
// BIAS / SILU / RMSNORM, with no scales: y = acc + bias.
enum EpiKind { EPI_BIAS = 0, EPI_SILU = 1, EPI_RMSNORM = 2, EPI_ACC = 3, EPI_PARTIAL = 4, EPI_F32BIAS = 5,
               EPI_F32SILU = 6, EPI_F32RMSNORM = 7 };

struct Plan {
    int tile;       // qdt_tile
    int bm, bn;     // token rows, weight rows per tile
    int tiles_m, tiles_n, split_k, kt_total, kt_per_split, grid, group_m;
    int64_t ws_bytes;
};

// Planner: pure host computation.  esize = operand bytes (1 int8, 2 bf16).
// tile_req / split_req: QDT_TILE_AUTO / 0 for automatic.
qdt_status make_plan(int64_t M, int64_t N, int64_t K, int epi, int esize, int tile_req, int split_req, Plan* p,
                     bool fp4 = false);

struct GemmArgs {
    const void* X;       // token operand [M][K] (int8 or bf16)
    const void* W;       // weight operand [N][K]
    const float* sx;     // [M] (int8 path)
    const float* sw;     // [N] (int8 path)
    const uint16_t* bias;
    const uint16_t* gamma;
    float eps;
    void* Y;
    int64_t ldy;
    int32_t* ws;         // split-K partials [S][M][N]
    uint64_t* clk;       // clock record of the GEMM kernel (4 words per workgroup) or null
    int M, N, K;         // K in elements
    int epi;             // EpiKind for the fused epilogue (EPI_PARTIAL when split)
};

hipError_t launch_gemm_i8(const GemmArgs& a, const Plan& p, hipStream_t st);
// Clock record of the W8A8 GEMM (diagnostic): the next `grid` 4-word entries of the armed record
// buffer, or null when the record is off or full.
uint64_t* clock_record_take(int grid);
hipError_t launch_gemm_bf16(const GemmArgs& a, const Plan& p, hipStream_t st);
// Block-scaled FP4 GEMM (256 x 256 tiles; a K split writes fp32 partials to a.ws): a.K is the element count; xsc / wsc the
// biased block exponents [M][K/32] / [N][K/32]; a.epi EPI_F32BIAS, EPI_F32SILU, EPI_F32RMSNORM or
// EPI_ACC (fp32 accumulators).
hipError_t launch_gemm_mx(const GemmArgs& a, const uint8_t* xsc, const uint8_t* wsc, const Plan& p, hipStream_t st);
// Weight-only block formats: quantizer of W [N, ldw] (first K columns) into codes Q and half
// scales D, and the linear Y = X * dequant(W)^T (+ bias) on bf16 matrix cores.  epi: EPI_F32BIAS
// (bf16 Y) or EPI_ACC (fp32 Y); a K split (pl.split_k > 1) writes fp32 partials to ws.
hipError_t launch_wo_quant(const uint16_t* W, int64_t ldw, int64_t N, int64_t K, int bits, uint8_t* Q, uint16_t* D,
                           hipStream_t st);
hipError_t launch_wo_gemm(const uint16_t* X, int64_t ldx, const uint8_t* Wq, const uint16_t* Wd, int bits,
                          const uint16_t* bias, int M, int N, int K, int epi, void* Y, int64_t ldy, float* ws,
                          const Plan& pl, hipStream_t st);
// Work layout of the attention: `tiles` (query block, head) tiles; the first t_full go to one
// workgroup each over all keys, each later one to `split` workgroups over key ranges (split 1 when
// there are none); `workgroups` in all; `part_floats` fp32 values of piece outputs; `vtr`: the PV
// product reads V transposed from LDS (S <= kAttnVtrMaxS), otherwise a V^T pass runs first.
constexpr int kAttnVtrMaxS = 8192;
struct AttnPlan {
    int tiles, t_full, split, workgroups;
    int64_t part_floats;
    bool vtr;
};
AttnPlan attention_plan(int S, int H);
// Softmax attention per 256-wide head: O = softmax(Q K^T / 16) V for every head; past
// kAttnVtrMaxS tokens V^T (keys permuted within 32-key groups, zero-padded to a multiple of 32
// keys) is written to Vt first (Vt unused otherwise).  redo: 4 ints per workgroup (one per wave,
// written on every call) for the exact-max rerun; part: the pieces' partial outputs
// (plan.part_floats floats, unused when the plan splits nothing).
hipError_t launch_attention(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int S, int H, int64_t ld,
                            uint16_t* O, int64_t ldo, uint16_t* Vt, int* redo, float* part, hipStream_t st);
// Sum of the S int32 partial slices followed by epilogue `epi` (BIAS, SILU, RMSNORM, ACC).
hipError_t launch_splitk_epilogue(const GemmArgs& a, int split_k, int epi, hipStream_t st);
// Sum of the S fp32 partial slices of the FP4 GEMM, then epilogue `epi` (F32BIAS, F32SILU,
// F32RMSNORM, ACC).
hipError_t launch_splitk_f32_epilogue(const GemmArgs& a, int split_k, int epi, hipStream_t st);

}  // namespace qdt
