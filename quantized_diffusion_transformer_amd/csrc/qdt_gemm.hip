// INT8 x INT8 -> INT32 GEMM on CDNA4 matrix cores with the dequantization epilogue fused,
// plus the bf16 GEMM of the protected (unquantized) layer on the same tile machinery.
//
// Method: "Quantizing a Dual-Branch Flow-Matching Diffusion Transformer for Consumer GPUs"
// (W8A8 recipe: acc = Xq . Wq^T with per-token and per-output-row scales; the FFN
// down-projection stays bf16).  Fused epilogues: "Serving sub-second Ideogram v4 without
// quality loss" (RMSNorm over 256-wide heads, gated SiLU kept on-chip).  Bias and row
// independence: "Faster Ideogram 4 with Less Prompt Compute", "Most of the Tensor Was Zero".
//
// Design (gfx950):
//   * One workgroup of 4 waves (one per SIMD) computes a BM x BN tile (256 x 256, or 288 x 288
//     where that makes the tile count a multiple of the 256 CUs); each wave owns an
//     (FM*16) x (FN*16) sub-tile as FN x FM accumulators of v_mfma_i32_16x16x64_i8
//     (v_mfma_f32_16x16x32_bf16 for bf16).  The MFMA A operand is the weight fragment and
//     the B operand the token fragment, so lane l holds 4 consecutive output columns of one
//     output row.
//   * K advances 128 bytes per stage (two MFMA K steps, whole cache lines) through two LDS
//     buffers filled by LDS-DMA (global_load_lds_dwordx4, no register staging); one barrier per
//     stage, between its two K steps.  LDS rows are XOR-swizzled so that the 16 rows read by
//     one ds_read_b128 fall in distinct banks.
//   * Tile order is XCD-aware: workgroup ids are dealt round-robin to the 8 XCDs, so ids are
//     remapped to give each XCD a contiguous run of tiles, walked in groups of `group_m` tile
//     rows, which keeps the operands of neighbouring tiles in that XCD's L2 (with split-K, the
//     K slice is the slowest index of the run).
//   * Epilogue parameters are staged in LDS during the prologue; outputs go through LDS strips
//     so that each store writes 16 contiguous bytes per lane.
//   * Rows beyond M (or N) are clamped loads whose outputs are not stored; the integer sum is
//     exact, so the result is independent of the tile shape and of the K split.
//   * Block-scaled FP4 (MXFP4) uses the same tiles: a 128-byte stage holds 256 FP4 elements,
//     exactly the bytes of two int8 K steps, and v_mfma_scale_f32_16x16x128_f8f6f4 reads its
//     fragments in the int8 layout.  Its per-lane block exponents (lane l covers the 32 elements
//     of one block) ride along in LDS: 8 bytes per row and stage, copied by dword LDS-DMAs with
//     the operand rows and read as single bytes beside the fragments.  The exponents are stored
//     stage-major (all rows' bytes of one 256-element stage together), so those LDS-DMAs read
//     whole cache lines.
#include <type_traits>

#include "qdt_device.h"
#include "qdt_internal.h"
#include "qdt_lds.h"

namespace qdt {

struct KArgs {
    const uint8_t* X;
    const uint8_t* W;
    const float* sx;
    const float* sw;
    const uint16_t* bias;
    const uint16_t* gamma;
    const uint8_t* xsc;  // block-scaled FP4: biased block exponents of X [M][K/32] and W [N][K/32]
    const uint8_t* wsc;
    void* Y;
    int32_t* ws;
    uint64_t* clk;       // clock record: 4 words per workgroup (start / end shader cycles and real time), or null
    int64_t ldy;
    float eps;
    int M, N, Kb, F;
    int tiles_m, tiles_n, split_k, kt_per_split, kt_total, group_m, head_dim;
};

template <bool BF16>
struct AccT;
template <>
struct AccT<false> { typedef v4i type; };
template <>
struct AccT<true> { typedef v4f type; };

// MFMA with the accumulator tied in place (dst == srcC).  Issued from inline asm: the
// compiler's own MFMA selection may pick the untied form, whose early-clobber destination
// forces accumulators to rotate through a spare register tuple on every iteration once all
// 256 accumulation registers are in use.  ACC_AGPR selects where the tuple lives (AGPR, or a
// VGPR tuple for tiles with more than 64 accumulator tuples per wave).  Being asm, these are
// invisible to the hazard recognizer: the kernel waits explicitly before reading accumulators.
template <bool BF16, bool ACC_AGPR>
__device__ __forceinline__ void mfma(typename AccT<BF16>::type& c, const v4u& a, const v4u& b) {
    if constexpr (BF16) {
        if constexpr (ACC_AGPR)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
        else
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
    } else {
        if constexpr (ACC_AGPR)
            asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
        else
            asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
    }
}

// Block-scaled FP4 MFMA, accumulator tied in place: A and B are 32 FP4 codes per lane (16 bytes,
// the int8 fragment layout), sa / sb hold the biased block exponents of the lane's A and B blocks
// in byte BYTE (0 or 1, chosen by op_sel; cbsz / blgp 4 select FP4 for both operands).
template <bool ACC_AGPR, int BYTE>
__device__ __forceinline__ void mfma_mx(v4f& c, const v4u& a, const v4u& b, uint32_t sa, uint32_t sb) {
    if constexpr (BYTE == 0) {
        if constexpr (ACC_AGPR)
            asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                         : "+a"(c) : "v"(a), "v"(b), "v"(sa), "v"(sb));
        else
            asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                         : "+v"(c) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    } else {
        if constexpr (ACC_AGPR)
            asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[1,1,0] op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                         : "+a"(c) : "v"(a), "v"(b), "v"(sa), "v"(sb));
        else
            asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[1,1,0] op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                         : "+v"(c) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    }
}

// WM x WN waves, FM x FN fragments of 16x16 per wave.  BF16: bf16 operands; MX: block-scaled FP4
// operands (both with fp32 accumulators); neither: int8 operands, int32 accumulators.
template <int WM, int WN, int FM, int FN, bool BF16, int EPI, bool MX = false>
__global__ __attribute__((amdgpu_flat_work_group_size(WM * WN * 64, WM * WN * 64), amdgpu_waves_per_eu(1, 1))) void
gemm_kernel(KArgs p) {
    constexpr int NW = WM * WN;            // waves
    constexpr int BM = WM * FM * 16;
    constexpr int BN = WN * FN * 16;
    constexpr int BK = 128;                // K bytes per stage: two MFMA K steps, whole cache lines
    constexpr int NB = 2;                  // LDS stages (double buffer)
    constexpr int ROWS = BN + BM;          // LDS rows per stage: weight rows, then token rows
    constexpr int STAGE = ROWS * BK;
    // 1 KiB LDS blocks (8 rows) per stage: waves 0 and 1 copy the weight rows (gate and up
    // halves for SILU), waves 2 and 3 the token rows, NIW / NIX LDS-DMA instructions each
    constexpr int NBW = BN / 8, NBX = BM / 8;
    constexpr int NIW = NBW / 2, NIX = NBX / 2;
    constexpr int NI = NIW > NIX ? NIW : NIX;  // LDS-DMA slots per wave per stage
    // FP4: dword LDS-DMAs carry the block exponents, 8 bytes per row and stage (the stage's 256
    // elements are 8 blocks), 32 rows per instruction.  A region of R rows (weight or token rows)
    // takes R / 32 of them, the first of its two waves ceil(R / 64), the second the rest; a wave
    // with fewer than NSC repeats its last one (the same bytes to the same place).  The gate and
    // up halves of SILU tiles are copied by their own waves.
    constexpr int NDW = BN / 32, NDX = BM / 32;
    constexpr int NSC = !MX ? 0 : ((NDW + 1) / 2 > (NDX + 1) / 2 ? (NDW + 1) / 2 : (NDX + 1) / 2);
    constexpr int NDMA = NI + NSC;
    static_assert(!MX || (BM % 32 == 0 && BN % 32 == 0 && !BF16 &&
                          (EPI == EPI_F32BIAS || EPI == EPI_F32SILU || EPI == EPI_F32RMSNORM || EPI == EPI_ACC ||
                           EPI == EPI_PARTIAL)),
                  "FP4: tiles of whole 32-row exponent blocks, fp32-accumulator epilogues");
    // The per-lane LDS-DMA offsets are held in registers, except for FP4 tiles of more than 256
    // rows, where the registers go to the block exponents and the offsets are recomputed per
    // instruction (a min and a multiply-add).
    constexpr bool VOFF_REGS = !(MX && NI > 16);
    constexpr int NACC_A = 64;             // accumulator tuples held in AGPRs (the rest in VGPRs)
    constexpr bool SILU = EPI == EPI_SILU || EPI == EPI_F32SILU;
    constexpr bool RMS = EPI == EPI_RMSNORM || EPI == EPI_F32RMSNORM;
    static_assert(WM == 2 && WN == 2 && NBW % 2 == 0 && NBX % 2 == 0, "two waves per operand region");
    static_assert(!SILU || (NIW * 8 == BN / 2 && FN % 2 == 0), "one weight wave per gate / up half");
    // MFMA slots between consecutive reads of sub-step 0 (3 for the 7 x 8 fragments of 224 x 256)
    constexpr int SP = (FN + FM) * 4 <= FN * FM ? 4 : 3;
    static_assert((FN + FM) * SP <= FN * FM, "sub-step 0 reads fit between its MFMAs");
    // sub-step 1 puts LDS-DMA q at slot floor(q FN FM / NI) and read q two slots later: distinct
    // slots inside the sub-step when the DMA slots are at least 3 apart and reads <= DMAs
    static_assert(FN * FM >= 3 * NDMA && FN + FM <= NDMA, "sub-step 1 LDS-DMAs and reads fit between its MFMAs");
    using Acc = typename AccT<BF16 || MX>::type;

    __shared__ __attribute__((aligned(1024))) uint8_t smem[NB * STAGE];
    constexpr int SCST = ROWS * 8;  // block-exponent bytes per stage (FP4)
    __shared__ __attribute__((aligned(16))) uint8_t smem_sc[MX ? NB * SCST : 16];
    __shared__ float red[RMS ? WN * BM : 1];
    // Epilogue parameters staged in LDS (dwords, each array padded to whole 64-lane DMA chunks):
    // w_scale per tile weight row, x_scale per tile token row, bias per weight row (bf16 pairs),
    // gamma per head column (bf16 pairs).
    constexpr bool HAS_SCALE = EPI == EPI_BIAS || EPI == EPI_SILU || EPI == EPI_RMSNORM;
    constexpr bool HAS_BIAS = HAS_SCALE || EPI == EPI_F32BIAS || EPI == EPI_F32SILU || EPI == EPI_F32RMSNORM;
    constexpr int P_SW = 0, N_SW = HAS_SCALE ? (BN + 63) / 64 * 64 : 0;
    constexpr int P_SX = P_SW + N_SW, N_SX = HAS_SCALE ? (BM + 63) / 64 * 64 : 0;
    constexpr int P_B = P_SX + N_SX, N_B = HAS_BIAS ? (BN / 2 + 63) / 64 * 64 : 0;
    constexpr int P_G = P_B + N_B, N_G = RMS ? 128 : 0;
    constexpr int P_BF = P_G + N_G, N_BF = HAS_BIAS ? (BN + 63) / 64 * 64 : 0;  // bias as fp32 (epilogue)
    constexpr int NPRM = P_BF + N_BF;
    __shared__ __attribute__((aligned(16))) uint32_t prm[NPRM > 0 ? NPRM : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WN, wm = wave / WN;
    // clock record (diagnostic, off unless armed): wave 0 reads the shader-clock counter and the
    // fixed 100 MHz real-time counter here and after its last store
    uint64_t clk_c0 = 0, clk_r0 = 0;
    if (p.clk != nullptr && wave == 0) {
        clk_c0 = __builtin_amdgcn_s_memtime();
        clk_r0 = __builtin_amdgcn_s_memrealtime();
    }

    // ---- workgroup id -> (tile, K slice), contiguous per XCD
    const int bid = blockIdx.x, nb = gridDim.x;
    const int xcd = bid % kNumXCD, per = nb / kNumXCD, rem = nb % kNumXCD;
    const int t = xcd * per + min(xcd, rem) + bid / kNumXCD;
    // K slice slowest: an XCD's run of workgroups covers one or two K slices of every tile, so
    // its L2 fetches the token rows of those slices only (with the slice fastest, every XCD
    // fetched every slice of X: 518 MB of L2 fills per 512 x 4608 x 53248 split-K-7 launch
    // instead of 304 MB)
    const int ntiles = p.tiles_m * p.tiles_n;
    const int split = t / ntiles;
    const int tt = t % ntiles;
    const int gsz = p.group_m * p.tiles_n;
    const int first_m = (tt / gsz) * p.group_m;
    const int gm = min(p.tiles_m - first_m, p.group_m);
    const int tm = first_m + (tt % gsz) % gm;
    const int tn = (tt % gsz) / gm;
    const int m0 = tm * BM;
    const int n0 = tn * (SILU ? BN / 2 : BN);  // first output column (SILU) / weight row
    const int kt0 = split * p.kt_per_split;
    const int kt1 = min(p.kt_total, kt0 + p.kt_per_split);
    const int nk = max(kt1 - kt0, 0);
    // first stage the LDS-DMAs address: an empty K slice still loads (unused) stage data from
    // inside the matrix, which keeps the prologue free of branches
    const int kta = min(kt0, p.kt_total - 1);

    // LDS rows are 128 bytes; chunk c of row g sits in slot c ^ (g & 7), which keeps the 16 rows
    // of a fragment read by one ds_read_b128 free of bank conflicts on gfx950 (measured with the
    // SQ_LDS_BANK_CONFLICT counter).

    // ---- LDS-DMA assignment: instruction i of wave w fills LDS block b = w * NI + i = tile rows
    // 8 b .. 8 b + 7 (weight rows first, then token rows); lane l moves row 8 b + l / 8, slot l % 8,
    // which holds global chunk (l % 8) ^ (row & 7).  A whole 128-byte line per row and stage:
    // half-line stages measured at 14 TB/s of L2 -> LDS traffic, whole lines at 21 TB/s.
    // Rows past the matrix end are clamped to its last row: their products only reach outputs
    // that are not stored.
    const int64_t Kb = p.Kb;
    const int nlim = SILU ? p.F : p.N;
    const int wlast = nlim - n0 - 1, xlast = p.M - m0 - 1;
    const int lchunk = (lane & 7) ^ ((lane >> 3) & 7);
    // The blocks of a wave lie in one operand region (weight rows; gate or up rows for SILU;
    // token rows): one scalar base per wave, a 32-bit offset per lane and instruction.
    const bool wwave = wave < 2;                 // weight-row wave
    const int niw = wwave ? NIW : NIX;           // its LDS-DMA instructions per stage
    const uint8_t* wbase;
    int rlocal0, rlast;
    if (wwave) {
        const bool up = SILU && wave == 1;
        wbase = p.W + (int64_t)((up ? p.F : 0) + n0) * Kb;
        rlocal0 = SILU ? 0 : wave * NIW * 8;
        rlast = wlast;
    } else {
        wbase = p.X + (int64_t)m0 * Kb;
        rlocal0 = (wave - 2) * NIX * 8;
        rlast = xlast;
    }
    wbase = uniform_ptr(wbase + (int64_t)kta * BK);
    // lane offset of LDS-DMA i: row rlocal0 + 8 i + lane / 8, clamped to the region's last row
    uint32_t voffs[VOFF_REGS ? NI : 1];
    int vrow = rlocal0 + (lane >> 3);  // recomputed offsets: lane row of instruction 0, chunk byte
    const uint32_t vch = lchunk * 16;
    if constexpr (VOFF_REGS) {
#pragma unroll
        for (int i = 0; i < NI; ++i) voffs[i] = (uint32_t)(min(vrow + i * 8, rlast) * Kb) + vch;
    }
    auto voff = [&](int i) __attribute__((always_inline)) {
        if constexpr (VOFF_REGS)
            return voffs[i];
        else
            return __umul24((uint32_t)min(vrow + i * 8, rlast), (uint32_t)Kb) + vch;
    };
    const int blk0 = wwave ? wave * NIW : NBW + (wave - 2) * NIX;  // first LDS block of the wave
    const uint32_t ldsw = __builtin_amdgcn_readfirstlane(lds_offset(smem) + blk0 * 1024);
    // whether LDS-DMA slot i is used by this wave (all are when both regions have equal rows)
    auto dma_used = [&](int i) __attribute__((always_inline)) { return NIW == NIX || i < niw; };
    // LDS-DMA instruction i of `stage` into LDS buffer `buf` (sets M0 itself)
    auto dma = [&](int buf, int stage, int i) __attribute__((always_inline)) {
        lds_dma16_s(ldsw + (uint32_t)(buf * STAGE + i * 1024), voff(i), wbase + (int64_t)stage * BK);
    };
    // FP4 block exponents, stored stage-major: for each 256-element stage, every row's 8 exponent
    // bytes are consecutive and rows follow each other (a stage's exponents of R rows are 8 R
    // contiguous bytes).  Dword LDS-DMA i of a wave copies rows erow0 + 32 i .. + 31 of its region
    // (lane l: row + l / 2, dword l % 2, i.e. 256 contiguous bytes) to LDS [row][8 bytes] of the
    // stage; instructions past the wave's ecnt repeat its last one.
    uint32_t scvoffs[NSC > 0 && VOFF_REGS ? NSC : 1];
    const uint8_t* scbase = nullptr;
    uint32_t ldss = 0;
    int64_t sstride = 0;  // exponent bytes per stage of the wave's operand (8 x its row count)
    int ecnt = 1, erow0 = 0;
    if constexpr (MX) {
        const int wrow0 = (SILU && wave == 1 ? p.F : 0) + n0;  // the up half's rows for SILU
        sstride = __builtin_amdgcn_readfirstlane(wwave ? p.N : p.M) * (int64_t)8;
        scbase = uniform_ptr((wwave ? p.wsc + (int64_t)wrow0 * 8 : p.xsc + (int64_t)m0 * 8) + (int64_t)kta * sstride);
        const bool first = (wave & 1) == 0;
        if (wwave && SILU) {
            ecnt = NDW / 2;
            erow0 = 0;
        } else {
            const int nd = wwave ? NDW : NDX;
            ecnt = first ? (nd + 1) / 2 : nd / 2;
            erow0 = first ? 0 : 32 * ((nd + 1) / 2);
        }
        const int row0 = wwave ? (SILU ? wave * (BN / 2) : erow0) : BN + erow0;
        ldss = __builtin_amdgcn_readfirstlane(lds_offset(smem_sc) + row0 * 8);
    }
    int erow = erow0 + (lane >> 1);  // lane row of exponent instruction 0
    const uint32_t edw = (lane & 1) * 4;
    auto scv = [&](int i) __attribute__((always_inline)) {
        return (uint32_t)(min(erow + i * 32, rlast) * 8) + edw;
    };
    if constexpr (MX && VOFF_REGS) {
#pragma unroll
        for (int i = 0; i < NSC; ++i) scvoffs[i] = scv(min(i, ecnt - 1));
    }
    // lane offset of exponent instruction i (already limited to ecnt - 1)
    auto scoff = [&](int i, int ie) __attribute__((always_inline)) {
        if constexpr (VOFF_REGS)
            return scvoffs[i];
        else
            return scv(ie);
    };
    auto sdma = [&](int buf, int stage, int i) __attribute__((always_inline)) {
        const int ie = min(i, ecnt - 1);
        lds_dma4_s(ldss + (uint32_t)(buf * SCST + ie * 256), scoff(i, ie), scbase + (int64_t)stage * sstride);
    };

    // Global weight row of tile weight row r (clamped like the operand rows).
    auto wglobal = [&](int r) __attribute__((always_inline)) {
        if constexpr (SILU) {
            const bool up = r >= BN / 2;
            return (up ? p.F : 0) + n0 + min(up ? r - BN / 2 : r, wlast);
        } else {
            return n0 + min(r, wlast);
        }
    };
    // Parameter DMA chunk c (64 dwords of prm), issued by wave c % NW.
    auto prm_dma = [&](int c) __attribute__((always_inline)) {
        const int e = c * 64 + lane;
        const void* src;
        if (e < P_SX) {
            src = p.sw + wglobal(min(e - P_SW, BN - 1));
        } else if (e < P_B) {
            src = p.sx + m0 + min(e - P_SX, min(BM - 1, xlast));
        } else if (e < P_G) {
            // pair of weight rows 2 q, 2 q + 1 (same half for SILU); clamping keeps pairs even
            const int r = 2 * min(e - P_B, BN / 2 - 1);
            int g;
            if constexpr (SILU) {
                const bool up = r >= BN / 2;
                g = (up ? p.F : 0) + n0 + min(up ? r - BN / 2 : r, wlast - 1);
            } else {
                g = n0 + min(r, wlast - 1);
            }
            src = p.bias + g;
        } else {
            src = p.gamma + 2 * min(e - P_G, 127);
        }
        lds_dma4(__builtin_amdgcn_readfirstlane(lds_offset(prm) + c * 256), src);
    };

    // ---- fragment reads: row (lane & 15) of a 16-row fragment, chunk 4 * ks + (lane >> 4)
    int wrow[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        if constexpr (SILU)
            wrow[fn] = fn < FN / 2 ? wn * (FN / 2) * 16 + fn * 16 : BN / 2 + wn * (FN / 2) * 16 + (fn - FN / 2) * 16;
        else
            wrow[fn] = wn * FN * 16 + fn * 16;
    }
    const int xrow0 = BN + wm * FM * 16;
    const int lrow = (lane & 15) * BK;
    const int lck0 = ((0 + (lane >> 4)) ^ (lane & 7)) << 4;
    const int lck1 = ((4 + (lane >> 4)) ^ (lane & 7)) << 4;

    Acc acc[FN][FM];

    // One MFMA of the group for weight fragment g, token fragment fm.
    auto mma = [&](int g, int fm, const v4u& a, const v4u& b) __attribute__((always_inline)) {
        if constexpr (!MX) {
            if (g * FM + fm < NACC_A)
                mfma<BF16, true>(acc[g][fm], a, b);
            else
                mfma<BF16, false>(acc[g][fm], a, b);
        }
    };
    // FP4: the block exponent of this lane's row (lane & 15) of a fragment starting at tile row
    // `row`, K step ks of the stage: lane group q = lane >> 4 covers block 4 ks + q, stored at byte
    // 2 q + ks of the row's 8 bytes
    // (both K steps' bytes of a block pair side by side: one 16-bit read gives the exponents of
    // K step 0 in byte 0 and of K step 1 in byte 1)
    const int sclane = (lane & 15) * 8 + 2 * (lane >> 4);
    auto sc16 = [&](int buf, int row) __attribute__((always_inline)) {
        return (uint32_t)*reinterpret_cast<const uint16_t*>(&smem_sc[buf * SCST + row * 8 + sclane]);
    };
    auto frag = [&](const uint8_t* s, int row, int lck) __attribute__((always_inline)) {
        return *reinterpret_cast<const v4u*>(s + row * BK + lck);
    };

    // ---- main loop over stages j = 0 .. nk-1 (stage j in LDS buffer j % 2), two MFMA K steps
    // (sub-steps) per stage.  The barrier sits between the sub-steps: when a wave reaches it, its
    // own LDS-DMAs of stage j+1 have landed (vmcnt 0) and its reads of stage j are complete (the
    // sub-step 1 fragments are in registers).  After it, stage j+1 is readable and buffer j % 2
    // is free, so sub-step 1 issues the LDS-DMAs of stage j+2 into buffer j % 2 and reads the
    // sub-step 0 fragments of stage j+1, while sub-step 0 reads the sub-step 1 fragments of its
    // own stage.  Every LDS read and LDS-DMA is issued between two MFMAs, so a wave never waits
    // on LDS latency after a barrier.  The last two stages are separate copies of the loop body:
    // they issue no LDS-DMAs (there is no stage j+2), and the last one reads no stage j+1, so after
    // its barrier no wave touches the stage buffers and the epilogue needs no barrier of its own.
    // Prologue: the LDS-DMAs of stage 0 go out first, then the parameter chunks (needed only by
    // the epilogue), then stage 1's; the accumulators are cleared while they are in flight.  Loads
    // complete in issue order, so vmcnt <= NI means stage 0 and the parameters have landed, and
    // the bias is converted to fp32 right after the first barrier.
    const int nkc = max(nk, 1);
    v4u a0[FN], b0[FM], a1[FN], b1[FM];
    // FP4 block exponents of the fragments for both K steps of a stage (byte 0: K step 0, byte 1:
    // K step 1).  ea[g] (weight fragment g) is used by row g of both sub-steps, so the next stage's
    // value is read into it right after row g of sub-step 1.  eb[fm] (token fragment fm) is used by
    // every row: sub-step 1 works from a copy, eb1, while the next stage's values are read into eb.
    uint32_t ea[MX ? FN : 1], eb[MX ? FM : 1], eb1[MX ? FM : 1];
    auto mmx = [&](int g, int fm, const v4u& a, const v4u& b, uint32_t sa, uint32_t sb, auto byte) __attribute__((always_inline)) {
        constexpr int BY = decltype(byte)::value;
        if constexpr (MX) {
            if (g * FM + fm < NACC_A)
                mfma_mx<true, BY>(acc[g][fm], a, b, sa, sb);
            else
                mfma_mx<false, BY>(acc[g][fm], a, b, sa, sb);
        } else {
            mma(g, fm, a, b);
        }
    };
#pragma unroll
    for (int i = 0; i < NI; ++i)
        if (dma_used(i)) dma(0, 0, i);
#pragma unroll
    for (int i = 0; i < NSC; ++i) sdma(0, 0, i);
    // the epilogue parameters land with stage 0 (loads complete in issue order)
#pragma unroll
    for (int c = 0; c < P_BF / 64; ++c) {
        const bool is_bias = c * 64 >= P_B && c * 64 < P_G;
        if (c % NW == wave && (!is_bias || p.bias != nullptr)) prm_dma(c);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
        if (dma_used(i)) dma(1, min(1, nkc - 1), i);
#pragma unroll
    for (int i = 0; i < NSC; ++i) sdma(1, min(1, nkc - 1), i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = Acc{0, 0, 0, 0};
    __builtin_amdgcn_sched_barrier(0);
    if (NIW == NIX)
        wait_vmcnt<NDMA>();
    else if (wwave)
        wait_vmcnt<NIW + NSC>();
    else
        wait_vmcnt<NIX + NSC>();
    __syncthreads();
    if constexpr (HAS_BIAS) {
        // bias of the tile's weight rows to fp32 (0 without bias), once; the main loop's barriers
        // order these writes before the epilogue reads them
        for (int r = tid; r < BN; r += NW * 64) {
            float v = 0.0f;
            if (p.bias) {
                const uint32_t pr = prm[P_B + r / 2];
                v = bf16_to_f32((r & 1) ? pr >> 16 : pr & 0xFFFFu);
            }
            prm[P_BF + r] = __float_as_uint(v);
        }
    }
    {
        const uint8_t* s = smem + lrow;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) a0[fn] = frag(s, wrow[fn], lck0);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) b0[fm] = frag(s, xrow0 + fm * 16, lck0);
        if constexpr (MX) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) ea[fn] = sc16(0, wrow[fn]);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) eb[fm] = sc16(0, xrow0 + fm * 16);
        }
    }
    // one main-loop stage; DMA: issue the LDS-DMAs of stage j + 2, NEXT: read the first fragments
    // of stage j + 1 (the last two stages have no stage j + 2, the last one no stage j + 1)
    auto iter = [&](int j, auto dma_on, auto next_on) __attribute__((always_inline)) {
        constexpr bool DMA = decltype(dma_on)::value, NEXT = decltype(next_on)::value;
        const uint8_t* s = smem + (j % NB) * STAGE + lrow;
        const uint8_t* sn = smem + ((j + 1) % NB) * STAGE + lrow;
        const int jd = j + 2;
        if constexpr (!VOFF_REGS) {
            // the recomputed LDS-DMA offsets stay inside the loop (hoisted, they would hold the
            // registers they are meant to free)
            asm volatile("" : "+v"(vrow));
            asm volatile("" : "+v"(erow));
        }
        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        // sub-step 0: every SP-th slot reads b1[0..FM-1], then a1[0..FN-1]
#pragma unroll
        for (int g = 0; g < FN; ++g) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                mmx(g, fm, a0[g], b0[fm], ea[MX ? g : 0], eb[MX ? fm : 0], B0{});
                const int k = g * FM + fm, q = k / SP;
                if (k % SP == 0 && q < FM)
                    b1[q] = frag(s, xrow0 + q * 16, lck1);
                else if (k % SP == 0 && q < FM + FN)
                    a1[q - FM] = frag(s, wrow[q - FM], lck1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_vmcnt<0>();
        __syncthreads();
        // sub-step 1: the LDS-DMAs of stage j+2 are spread evenly over the sub-step's MFMA slots
        // (each points M0 at the next one); two slots after LDS-DMA slot q, read q of stage j+1
        // (b0[q], then a0[q - FM])
        const uint32_t ldsd = ldsw + (uint32_t)((j % NB) * STAGE);
        const uint8_t* sbase = wbase + (int64_t)jd * BK;
        const uint32_t ldssd = ldss + (uint32_t)((j % NB) * SCST);
        const uint8_t* scbased = MX ? scbase + (int64_t)jd * sstride : nullptr;
        (void)ldssd;
        (void)scbased;
        if constexpr (MX) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) eb1[fm] = eb[fm];
        }
        if constexpr (DMA) set_m0(MX ? ldssd : ldsd);
#pragma unroll
        for (int g = 0; g < FN; ++g) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                mmx(g, fm, a1[g], b1[fm], ea[MX ? g : 0], eb1[MX ? fm : 0], B1{});
                const int k = g * FM + fm;
                // LDS-DMA q at slot floor(q * S / NDMA), read q two slots later (FP4: the next
                // stage's token-fragment exponents one slot later); the FP4 exponent LDS-DMAs
                // follow the operand ones
                constexpr int S = FN * FM;
                int qd = -1, qr = -1, qs = -1;
#pragma unroll
                for (int t = 0; t < NDMA; ++t) if ((t * S) / NDMA == k) qd = t;
#pragma unroll
                for (int t = 0; t < FM + FN; ++t) if ((t * S) / NDMA + 2 == k) qr = t;
#pragma unroll
                for (int t = 0; t < FM; ++t) if ((t * S) / NDMA + 1 == k) qs = t;
                // FP4: the exponent LDS-DMAs go first (they and the operand ones land before the next
                // barrier; the earliest slots leave them the most time)
                const int qop = MX ? qd - NSC : qd;  // operand LDS-DMA of this slot, if any
                if (qd >= 0 && qop >= 0) {
                    const uint32_t next = ldsd + (uint32_t)((qop + 1) * 1024);
                    if (DMA && dma_used(qop)) lds_dma16_next(voff(qop), sbase, next);
                } else if (qd >= 0) {
                    if constexpr (MX && DMA) {
                        const int i = qd, ie = min(i, ecnt - 1), inext = min(i + 1, ecnt - 1);
                        lds_dma4_next(scoff(i, ie), scbased, i + 1 < NSC ? ldssd + (uint32_t)(inext * 256) : ldsd);
                    }
                } else if (NEXT && qr >= 0 && qr < FM)
                    b0[qr] = frag(sn, xrow0 + qr * 16, lck0);
                else if (NEXT && qr >= FM)
                    a0[qr - FM] = frag(sn, wrow[qr - FM], lck0);
                if constexpr (MX && NEXT) {
                    if (qs >= 0) eb[qs] = sc16((j + 1) % NB, xrow0 + qs * 16);
                    // weight fragment g's exponents once row g is done: after the second MFMA of
                    // row g + 1, and the last row's after the sub-step's last MFMA
                    if (g >= 1 && fm == 1) ea[g - 1] = sc16((j + 1) % NB, wrow[g - 1]);
                    if (g == FN - 1 && fm == FM - 1) ea[FN - 1] = sc16((j + 1) % NB, wrow[FN - 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    using T = std::true_type;
    using F = std::false_type;
    for (int j = 0; j < nk - 2; ++j) iter(j, T{}, T{});
    if (nk >= 2) iter(nk - 2, F{}, T{});
    if (nk >= 1) iter(nk - 1, F{}, F{});
    wait_vmcnt<0>();
    mfma_drain();
#pragma unroll
    for (int g = 0; g < FN; ++g)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            if (g * FM + fm < NACC_A)
                keep_after_a(acc[g][fm]);
            else
                keep_after_v(acc[g][fm]);
        }

    // ---------------------------------------------------------------- epilogues
    // Staged parameters of tile weight rows rl .. rl+3 and tile token row.
    auto prm_sw4 = [&](int rl) __attribute__((always_inline)) { return *reinterpret_cast<const float4*>(&prm[P_SW + rl]); };
    auto prm_b4 = [&](int rl, float (&b)[4]) __attribute__((always_inline)) {
        const float4 v = *reinterpret_cast<const float4*>(&prm[P_BF + rl]);
        b[0] = v.x; b[1] = v.y; b[2] = v.z; b[3] = v.w;
    };
    auto prm_sx = [&](int rt) __attribute__((always_inline)) { return __uint_as_float(prm[P_SX + rt]); };
    const int ncol0 = wn * (SILU ? FN / 2 : FN) * 16 + 4 * (lane >> 4);  // + fn * 16: tile weight row

    // ---- output through LDS.  Per 16-row strip (one fm) a wave writes its fragments to a private
    // LDS strip in row-major order and reads them back 16 bytes per lane, so each global store
    // writes whole row segments instead of 16 rows x 32 bytes.  The stage buffers are reused
    // (after a barrier: other waves may still read the last stage); two strips per wave alternate.
    constexpr int NF = SILU ? FN / 2 : FN;                               // output fragments per row
    constexpr int ES = (EPI == EPI_ACC || EPI == EPI_PARTIAL) ? 4 : 2;   // output element bytes
    constexpr int CW = NF * 16 * ES, RS = CW + 16, CPR = CW / 16, NCH = 16 * CPR;
    static_assert(NW * 2 * 16 * RS <= NB * STAGE, "output strips fit in the stage buffers");
    // no barrier: after the last stage's barrier no wave reads the stage buffers, no LDS-DMA is in
    // flight, and each wave's output strips are its own
    uint8_t* Yb;
    int64_t ldb;
    int ncols;
    if constexpr (EPI == EPI_PARTIAL) {
        Yb = reinterpret_cast<uint8_t*>(p.ws + (int64_t)split * p.M * p.N);
        ldb = (int64_t)p.N * 4;
        ncols = p.N;
    } else {
        Yb = reinterpret_cast<uint8_t*>(p.Y);
        ldb = p.ldy * ES;
        ncols = SILU ? p.F : p.N;
    }
    const int colw = n0 + wn * NF * 16;  // first output column of the wave
    // Read-back chunk it of a lane: strip row r_it, 16-byte column chunk cc_it (the same in every
    // strip, so the offsets are computed once).
    constexpr int NIT = (NCH + 63) / 64;
    int rr[NIT], lofs[NIT];
    int64_t gofs[NIT];
    bool ok[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int c = it * 64 + lane, r = c / CPR, cc = c % CPR, n = colw + cc * (16 / ES);
        rr[it] = r;
        lofs[it] = r * RS + cc * 16;
        gofs[it] = (int64_t)r * ldb + (int64_t)n * ES;
        ok[it] = (NCH % 64 == 0 || c < NCH) && n < ncols;
    }
    // Strip fm: the lane's 4 outputs of fragment (fn, fm) (frag_out(fn)) go to row lane & 15 of the
    // LDS strip, columns fn * 16 + 4 * (lane >> 4) .. + 3.  Strips alternate between two LDS
    // buffers and are software-pipelined: strip fm is written, then strip fm - 1 is read back and
    // stored.  The LDS executes one wave's instructions in order, so a read-back sees the same
    // wave's earlier strip writes (and strip fm - 1 was written a whole strip of work earlier);
    // strip fm + 1 overwrites strip fm - 1's buffer only after the stores that consumed its
    // read-back.  The asm statements are compiler barriers that keep this order.
    auto store_strip = [&](int fm) __attribute__((always_inline)) {
        const uint8_t* st = smem + (wave * 2 + (fm & 1)) * 16 * RS;
        uint8_t* yrow = Yb + (int64_t)(m0 + wm * FM * 16 + fm * 16) * ldb;
        const int rows_left = p.M - (m0 + wm * FM * 16 + fm * 16);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const v4u v = *reinterpret_cast<const v4u*>(st + lofs[it]);
            if (ok[it] && rr[it] < rows_left) {
                v4u* dst = reinterpret_cast<v4u*>(yrow + gofs[it]);
                // the output is consumed by a later kernel: stream it past the caches (measured
                // faster for back-to-back linears); split-K partials are re-read at once, cached
                if constexpr (EPI == EPI_PARTIAL)
                    *dst = v;
                else
                    __builtin_nontemporal_store(v, dst);
            }
        }
    };
    auto put_strip = [&](int fm, auto&& frag_out) __attribute__((always_inline)) {
        // one strip at a time: keeps the scheduler from hoisting every accumulator read (and
        // spilling) ahead of the first store
        __builtin_amdgcn_sched_barrier(0);
        uint8_t* st = smem + (wave * 2 + (fm & 1)) * 16 * RS;
#pragma unroll
        for (int fn = 0; fn < NF; ++fn) {
            const auto v = frag_out(fn);
            *reinterpret_cast<std::remove_const_t<decltype(v)>*>(st + (lane & 15) * RS + (fn * 16 + 4 * (lane >> 4)) * ES) = v;
        }
        if (fm > 0) {
            asm volatile("" ::: "memory");
            store_strip(fm - 1);
        }
        if (fm == FM - 1) {
            asm volatile("" ::: "memory");
            store_strip(fm);
        }
    };
    auto prm_sxf = [&](int fm) __attribute__((always_inline)) { return prm_sx(wm * FM * 16 + fm * 16 + (lane & 15)); };

    if constexpr (EPI == EPI_ACC || EPI == EPI_PARTIAL) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) put_strip(fm, [&](int fn) { return acc[fn][fm]; });
    } else if constexpr (EPI == EPI_F32BIAS) {
        float b[FN][4];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) prm_b4(ncol0 + fn * 16, b[fn]);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            put_strip(fm, [&](int fn) {
                const Acc& a = acc[fn][fm];
                return make_uint2(pack_bf16x2((float)a[0] + b[fn][0], (float)a[1] + b[fn][1]),
                                  pack_bf16x2((float)a[2] + b[fn][2], (float)a[3] + b[fn][3]));
            });
    } else if constexpr (EPI == EPI_BIAS) {
        float4 sw[FN];
        float b[FN][4];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            sw[fn] = prm_sw4(ncol0 + fn * 16);
            prm_b4(ncol0 + fn * 16, b[fn]);
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const float sx = prm_sxf(fm);
            put_strip(fm, [&](int fn) {
                const Acc& a = acc[fn][fm];
                return make_uint2(pack_bf16x2(dequant(a[0], sx, sw[fn].x, b[fn][0]), dequant(a[1], sx, sw[fn].y, b[fn][1])),
                                  pack_bf16x2(dequant(a[2], sx, sw[fn].z, b[fn][2]), dequant(a[3], sx, sw[fn].w, b[fn][3])));
            });
        }
    } else if constexpr (EPI == EPI_SILU) {
        // gate fragment fn pairs with up fragment fn + FN / 2 (tile weight rows BN / 2 further)
        float swg[NF][4], swu[NF][4], bg[NF][4], bu[NF][4];
#pragma unroll
        for (int fn = 0; fn < NF; ++fn) {
            const int rl = ncol0 + fn * 16;
            const float4 g4 = prm_sw4(rl), u4 = prm_sw4(BN / 2 + rl);
            swg[fn][0] = g4.x; swg[fn][1] = g4.y; swg[fn][2] = g4.z; swg[fn][3] = g4.w;
            swu[fn][0] = u4.x; swu[fn][1] = u4.y; swu[fn][2] = u4.z; swu[fn][3] = u4.w;
            prm_b4(rl, bg[fn]);
            prm_b4(BN / 2 + rl, bu[fn]);
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const float sx = prm_sxf(fm);
            put_strip(fm, [&](int fn) {
                float g[4], u[4], y[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    g[r] = dequant(acc[fn][fm][r], sx, swg[fn][r], bg[fn][r]);
                    u[r] = dequant(acc[fn + NF][fm][r], sx, swu[fn][r], bu[fn][r]);
                }
                silu_gate4(g, u, y);
                return make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
            });
        }
    } else if constexpr (EPI == EPI_F32SILU) {
        // fp32 accumulators (block-scaled FP4): g = acc_g + b_g, u = acc_u + b_u, y = silu(g) u
        float bg[NF][4], bu[NF][4];
#pragma unroll
        for (int fn = 0; fn < NF; ++fn) {
            const int rl = ncol0 + fn * 16;
            prm_b4(rl, bg[fn]);
            prm_b4(BN / 2 + rl, bu[fn]);
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            put_strip(fm, [&](int fn) {
                float g[4], u[4], y[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    g[r] = (float)acc[fn][fm][r] + bg[fn][r];
                    u[r] = (float)acc[fn + NF][fm][r] + bu[fn][r];
                }
                silu_gate4(g, u, y);
                return make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
            });
        }
    } else if constexpr (RMS) {
        // The workgroup's BN = 256 columns are exactly one head; each wave holds FN*16 of
        // them, so a head spans the fragments of WN waves.  Row sums of y^2: in-lane over
        // fragments, across the 4 lane groups with shuffles, across waves through LDS, in a
        // fixed order.
        static_assert(BN == 256, "one head per tile");
        // y: the dequantized output plus bias (int8), or the fp32 accumulator plus bias (FP4)
        constexpr bool F32 = EPI == EPI_F32RMSNORM;
        float sxv[FM], ss[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            sxv[fm] = F32 ? 0.0f : prm_sxf(fm);
            ss[fm] = 0.0f;
        }
        float swv[FN][4], bv[FN][4];
        auto yv = [&](int fn, int fm, int r) __attribute__((always_inline)) {
            if constexpr (F32)
                return (float)acc[fn][fm][r] + bv[fn][r];
            else
                return dequant(acc[fn][fm][r], sxv[fm], swv[fn][r], bv[fn][r]);
        };
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            if constexpr (!F32) {
                const float4 sw = prm_sw4(ncol0 + fn * 16);
                swv[fn][0] = sw.x; swv[fn][1] = sw.y; swv[fn][2] = sw.z; swv[fn][3] = sw.w;
            }
            prm_b4(ncol0 + fn * 16, bv[fn]);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float y = yv(fn, fm, r);
                    ss[fm] += y * y;
                }
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            ss[fm] += __shfl_xor(ss[fm], 16, 64);
            ss[fm] += __shfl_xor(ss[fm], 32, 64);
            if ((lane >> 4) == 0) red[wn * BM + wm * FM * 16 + fm * 16 + lane] = ss[fm];
        }
        __syncthreads();
        float rinv[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int rl = wm * FM * 16 + fm * 16 + (lane & 15);
            float tot = red[rl];
#pragma unroll
            for (int w = 1; w < WN; ++w) tot += red[w * BM + rl];
            const float ms = tot / (float)p.head_dim;
            rinv[fm] = 1.0f / sqrtf(ms + p.eps);
        }
        float g[FN][4];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const uint2 gg = *reinterpret_cast<const uint2*>(&prm[P_G + (ncol0 + fn * 16) / 2]);  // column within the head
            g[fn][0] = bf16_to_f32(gg.x & 0xFFFFu); g[fn][1] = bf16_to_f32(gg.x >> 16);
            g[fn][2] = bf16_to_f32(gg.y & 0xFFFFu); g[fn][3] = bf16_to_f32(gg.y >> 16);
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            put_strip(fm, [&](int fn) {
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float y = yv(fn, fm, r);
                    o[r] = (y * rinv[fm]) * g[fn][r];
                }
                return make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            });
    }
    if (p.clk != nullptr && wave == 0) {
        const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
        if (lane == 0) {
            uint64_t* o = p.clk + 4 * (int64_t)blockIdx.x;
            o[0] = clk_c0;
            o[1] = clk_r0;
            o[2] = c1;
            o[3] = r1;
        }
    }
}

// ---------------------------------------------------------------------------- split-K epilogue
// Sum of y^2 over one 256-wide head, in exactly the order of the fused RMSNorm epilogue, so that
// a split plan gives the same bits as the fused one.  Lane L of the wave holds columns 4L .. 4L+3
// of the head (y[0..3]).  In the fused kernel the head is split between two waves of 128 columns;
// there lane group q (lanes 16q .. 16q+15 of a fragment row) sums the squares of columns
// 128 wn + 16 fn + 4 q + r in the order fn = 0..7, r = 0..3; the four lane-group sums are combined
// as (P0 + P1) + (P2 + P3) and the two waves' totals as T0 + T1.  Here that column is held by
// lane 32 wn + 4 fn + q.
__device__ __forceinline__ float head_sumsq_fused_order(const float (&y)[4], int lane) {
    float sq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sq[r] = y[r] * y[r];
    const int base = (lane & 32) | (lane & 3);
    float p = 0.0f;
#pragma unroll
    for (int fn = 0; fn < 8; ++fn)
#pragma unroll
        for (int r = 0; r < 4; ++r) p += __shfl(sq[r], base | (fn << 2), 64);
    p += __shfl_xor(p, 1, 64);
    p += __shfl_xor(p, 2, 64);
    return __shfl(p, 0, 64) + __shfl(p, 32, 64);
}

// Sums the S int32 partial slices (exact, any order) and applies the same epilogue
// arithmetic as the fused kernel, including its order of the head RMSNorm's sum of squares, so
// every plan gives the same bits.  BIAS / SILU / ACC: one thread per 4 output columns; RMSNORM:
// one wave per (row, head).
template <int EPI>
__global__ __launch_bounds__(256) void splitk_epi_kernel(KArgs p) {
    const int64_t MN = (int64_t)p.M * p.N;
    if constexpr (EPI == EPI_RMSNORM) {
        // one wave per (row, head): 64 lanes x 4 columns
        const int heads = p.N / p.head_dim;
        const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
        if (item >= (int64_t)p.M * heads) return;
        const int lane = threadIdx.x & 63;
        const int m = (int)(item / heads), h = (int)(item % heads);
        const int d = lane * 4, n = h * p.head_dim + d;
        v4i a = *reinterpret_cast<const v4i*>(p.ws + (int64_t)m * p.N + n);
        for (int s = 1; s < p.split_k; ++s) a += *reinterpret_cast<const v4i*>(p.ws + s * MN + (int64_t)m * p.N + n);
        const float sx = p.sx[m];
        const float4 sw = *reinterpret_cast<const float4*>(p.sw + n);
        const float swv[4] = {sw.x, sw.y, sw.z, sw.w};
        float b[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.bias) {
            uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
            b[0] = bf16_to_f32(bb.x & 0xFFFFu); b[1] = bf16_to_f32(bb.x >> 16);
            b[2] = bf16_to_f32(bb.y & 0xFFFFu); b[3] = bf16_to_f32(bb.y >> 16);
        }
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = dequant(a[r], sx, swv[r], b[r]);
        const float ss = head_sumsq_fused_order(y, lane);
        const float ms = ss / (float)p.head_dim;
        const float rinv = 1.0f / sqrtf(ms + p.eps);
        uint2 gg = *reinterpret_cast<const uint2*>(p.gamma + d);
        const float g[4] = {bf16_to_f32(gg.x & 0xFFFFu), bf16_to_f32(gg.x >> 16), bf16_to_f32(gg.y & 0xFFFFu),
                            bf16_to_f32(gg.y >> 16)};
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = (y[r] * rinv) * g[r];
        uint16_t* Y = reinterpret_cast<uint16_t*>(p.Y);
        *reinterpret_cast<uint2*>(Y + (int64_t)m * p.ldy + n) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    } else {
        const int nout = EPI == EPI_SILU ? p.F : p.N;
        const int q = nout / 4;
        const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
        if (idx >= (int64_t)p.M * q) return;
        const int m = (int)(idx / q);
        const int n = (int)(idx % q) * 4;
        v4i a = *reinterpret_cast<const v4i*>(p.ws + (int64_t)m * p.N + n);
        for (int s = 1; s < p.split_k; ++s) a += *reinterpret_cast<const v4i*>(p.ws + s * MN + (int64_t)m * p.N + n);
        if constexpr (EPI == EPI_ACC) {
            *reinterpret_cast<v4i*>(reinterpret_cast<int32_t*>(p.Y) + (int64_t)m * p.ldy + n) = a;
            return;
        }
        const float sx = p.sx[m];
        const float4 sw = *reinterpret_cast<const float4*>(p.sw + n);
        const float swv[4] = {sw.x, sw.y, sw.z, sw.w};
        float b[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.bias) {
            uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
            b[0] = bf16_to_f32(bb.x & 0xFFFFu); b[1] = bf16_to_f32(bb.x >> 16);
            b[2] = bf16_to_f32(bb.y & 0xFFFFu); b[3] = bf16_to_f32(bb.y >> 16);
        }
        float y[4];
        if constexpr (EPI == EPI_SILU) {
            v4i u = *reinterpret_cast<const v4i*>(p.ws + (int64_t)m * p.N + p.F + n);
            for (int s = 1; s < p.split_k; ++s)
                u += *reinterpret_cast<const v4i*>(p.ws + s * MN + (int64_t)m * p.N + p.F + n);
            const float4 swu = *reinterpret_cast<const float4*>(p.sw + p.F + n);
            const float swuv[4] = {swu.x, swu.y, swu.z, swu.w};
            float bu[4] = {0.f, 0.f, 0.f, 0.f};
            if (p.bias) {
                uint2 bb = *reinterpret_cast<const uint2*>(p.bias + p.F + n);
                bu[0] = bf16_to_f32(bb.x & 0xFFFFu); bu[1] = bf16_to_f32(bb.x >> 16);
                bu[2] = bf16_to_f32(bb.y & 0xFFFFu); bu[3] = bf16_to_f32(bb.y >> 16);
            }
            float gg[4], uu[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                gg[r] = dequant(a[r], sx, swv[r], b[r]);
                uu[r] = dequant(u[r], sx, swuv[r], bu[r]);
            }
            silu_gate4(gg, uu, y);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = dequant(a[r], sx, swv[r], b[r]);
        }
        uint16_t* Y = reinterpret_cast<uint16_t*>(p.Y);
        *reinterpret_cast<uint2*>(Y + (int64_t)m * p.ldy + n) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
    }
}

// ---------------------------------------------------------------------------- launchers
static KArgs make_kargs(const GemmArgs& a, const Plan& pl, int esize) {
    KArgs k;
    k.X = reinterpret_cast<const uint8_t*>(a.X);
    k.W = reinterpret_cast<const uint8_t*>(a.W);
    k.sx = a.sx;
    k.sw = a.sw;
    k.bias = a.bias;
    k.gamma = a.gamma;
    k.Y = a.Y;
    k.ws = a.ws;
    k.ldy = a.ldy;
    k.eps = a.eps;
    k.M = a.M;
    k.N = a.N;
    k.Kb = a.K * esize;
    k.F = a.N / 2;
    k.tiles_m = pl.tiles_m;
    k.tiles_n = pl.tiles_n;
    k.split_k = pl.split_k;
    k.kt_per_split = pl.kt_per_split;
    k.kt_total = pl.kt_total;
    k.group_m = pl.group_m;
    k.head_dim = 256;
    k.xsc = nullptr;
    k.wsc = nullptr;
    k.clk = a.clk;
    return k;
}

template <int FM, int FN, bool BF16, int EPI, bool MX = false>
static hipError_t go(const KArgs& k, int grid, hipStream_t st) {
    hipLaunchKernelGGL((gemm_kernel<2, 2, FM, FN, BF16, EPI, MX>), dim3(grid), dim3(256), 0, st, k);
    return hipGetLastError();
}

hipError_t launch_gemm_i8(const GemmArgs& a, const Plan& pl, hipStream_t st) {
    KArgs k = make_kargs(a, pl, 1);
    const int epi = pl.split_k > 1 ? EPI_PARTIAL : a.epi;
    if (pl.tile == QDT_TILE_288) {
        switch (epi) {
            case EPI_BIAS: return go<9, 9, false, EPI_BIAS>(k, pl.grid, st);
            case EPI_ACC: return go<9, 9, false, EPI_ACC>(k, pl.grid, st);
            case EPI_PARTIAL: return go<9, 9, false, EPI_PARTIAL>(k, pl.grid, st);
            default: return hipErrorInvalidValue;
        }
    }
    if (pl.tile == QDT_TILE_224x256) {
        switch (epi) {
            case EPI_BIAS: return go<7, 8, false, EPI_BIAS>(k, pl.grid, st);
            case EPI_SILU: return go<7, 8, false, EPI_SILU>(k, pl.grid, st);
            case EPI_RMSNORM: return go<7, 8, false, EPI_RMSNORM>(k, pl.grid, st);
            case EPI_ACC: return go<7, 8, false, EPI_ACC>(k, pl.grid, st);
            case EPI_PARTIAL: return go<7, 8, false, EPI_PARTIAL>(k, pl.grid, st);
            default: return hipErrorInvalidValue;
        }
    }
    if (pl.tile == QDT_TILE_288x256) {
        switch (epi) {
            case EPI_BIAS: return go<9, 8, false, EPI_BIAS>(k, pl.grid, st);
            case EPI_SILU: return go<9, 8, false, EPI_SILU>(k, pl.grid, st);
            case EPI_RMSNORM: return go<9, 8, false, EPI_RMSNORM>(k, pl.grid, st);
            case EPI_ACC: return go<9, 8, false, EPI_ACC>(k, pl.grid, st);
            case EPI_PARTIAL: return go<9, 8, false, EPI_PARTIAL>(k, pl.grid, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (epi) {
        case EPI_BIAS: return go<8, 8, false, EPI_BIAS>(k, pl.grid, st);
        case EPI_SILU: return go<8, 8, false, EPI_SILU>(k, pl.grid, st);
        case EPI_RMSNORM: return go<8, 8, false, EPI_RMSNORM>(k, pl.grid, st);
        case EPI_ACC: return go<8, 8, false, EPI_ACC>(k, pl.grid, st);
        case EPI_PARTIAL: return go<8, 8, false, EPI_PARTIAL>(k, pl.grid, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_bf16(const GemmArgs& a, const Plan& pl, hipStream_t st) {
    KArgs k = make_kargs(a, pl, 2);
    if (pl.tile == QDT_TILE_288) return go<9, 9, true, EPI_F32BIAS>(k, pl.grid, st);
    if (pl.tile == QDT_TILE_288x256) return go<9, 8, true, EPI_F32BIAS>(k, pl.grid, st);
    return go<8, 8, true, EPI_F32BIAS>(k, pl.grid, st);
}

hipError_t launch_gemm_mx(const GemmArgs& a, const uint8_t* xsc, const uint8_t* wsc, const Plan& pl, hipStream_t st) {
    KArgs k = make_kargs(a, pl, 1);
    k.Kb = a.K / 2;  // two FP4 codes per byte
    k.xsc = xsc;
    k.wsc = wsc;
    const int epi = pl.split_k > 1 ? EPI_PARTIAL : a.epi;
    if (pl.tile == QDT_TILE_288) {
        switch (epi) {
            case EPI_F32BIAS: return go<9, 9, false, EPI_F32BIAS, true>(k, pl.grid, st);
            case EPI_ACC: return go<9, 9, false, EPI_ACC, true>(k, pl.grid, st);
            case EPI_PARTIAL: return go<9, 9, false, EPI_PARTIAL, true>(k, pl.grid, st);
            default: return hipErrorInvalidValue;
        }
    }
    if (pl.tile == QDT_TILE_288x256) {
        switch (epi) {
            case EPI_F32BIAS: return go<9, 8, false, EPI_F32BIAS, true>(k, pl.grid, st);
            case EPI_F32SILU: return go<9, 8, false, EPI_F32SILU, true>(k, pl.grid, st);
            case EPI_F32RMSNORM: return go<9, 8, false, EPI_F32RMSNORM, true>(k, pl.grid, st);
            case EPI_ACC: return go<9, 8, false, EPI_ACC, true>(k, pl.grid, st);
            case EPI_PARTIAL: return go<9, 8, false, EPI_PARTIAL, true>(k, pl.grid, st);
            default: return hipErrorInvalidValue;
        }
    }
    if (pl.tile != QDT_TILE_256) return hipErrorInvalidValue;
    switch (epi) {
        case EPI_F32BIAS: return go<8, 8, false, EPI_F32BIAS, true>(k, pl.grid, st);
        case EPI_F32SILU: return go<8, 8, false, EPI_F32SILU, true>(k, pl.grid, st);
        case EPI_F32RMSNORM: return go<8, 8, false, EPI_F32RMSNORM, true>(k, pl.grid, st);
        case EPI_ACC: return go<8, 8, false, EPI_ACC, true>(k, pl.grid, st);
        case EPI_PARTIAL: return go<8, 8, false, EPI_PARTIAL, true>(k, pl.grid, st);
        default: return hipErrorInvalidValue;
    }
}

// Block-scaled FP4 split-K: sums the S fp32 partial slices in slice order and applies the
// fp32-accumulator epilogues to y = sum + bias (the same functions as the fused kernel).
// F32BIAS / F32SILU / ACC: one thread per 4 output columns; F32RMSNORM: one wave per (row, head).
template <int EPI>
__global__ __launch_bounds__(256) void splitk_f32_epi_kernel(KArgs p) {
    const int64_t MN = (int64_t)p.M * p.N;
    const float* ws = reinterpret_cast<const float*>(p.ws);
    auto sum4 = [&](int64_t off) __attribute__((always_inline)) {
        v4f a = *reinterpret_cast<const v4f*>(ws + off);
        for (int s = 1; s < p.split_k; ++s) a += *reinterpret_cast<const v4f*>(ws + s * MN + off);
        return a;
    };
    auto bias4 = [&](int n, float (&b)[4]) __attribute__((always_inline)) {
        b[0] = b[1] = b[2] = b[3] = 0.0f;
        if (p.bias) {
            const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
            b[0] = bf16_to_f32(bb.x & 0xFFFFu); b[1] = bf16_to_f32(bb.x >> 16);
            b[2] = bf16_to_f32(bb.y & 0xFFFFu); b[3] = bf16_to_f32(bb.y >> 16);
        }
    };
    uint16_t* Y = reinterpret_cast<uint16_t*>(p.Y);
    if constexpr (EPI == EPI_F32RMSNORM) {
        const int heads = p.N / p.head_dim;
        const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
        if (item >= (int64_t)p.M * heads) return;
        const int lane = threadIdx.x & 63;
        const int m = (int)(item / heads), h = (int)(item % heads);
        const int d = lane * 4, n = h * p.head_dim + d;
        const v4f a = sum4((int64_t)m * p.N + n);
        float b[4], y[4];
        bias4(n, b);
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = a[r] + b[r];
        const float ss = head_sumsq_fused_order(y, lane);
        const float rinv = 1.0f / sqrtf(ss / (float)p.head_dim + p.eps);
        const uint2 gg = *reinterpret_cast<const uint2*>(p.gamma + d);
        const float g[4] = {bf16_to_f32(gg.x & 0xFFFFu), bf16_to_f32(gg.x >> 16), bf16_to_f32(gg.y & 0xFFFFu),
                            bf16_to_f32(gg.y >> 16)};
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = (y[r] * rinv) * g[r];
        *reinterpret_cast<uint2*>(Y + (int64_t)m * p.ldy + n) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    } else {
        const int nout = EPI == EPI_F32SILU ? p.F : p.N;
        const int q = nout / 4;
        const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
        if (idx >= (int64_t)p.M * q) return;
        const int m = (int)(idx / q);
        const int n = (int)(idx % q) * 4;
        const v4f a = sum4((int64_t)m * p.N + n);
        if constexpr (EPI == EPI_ACC) {
            *reinterpret_cast<v4f*>(reinterpret_cast<float*>(p.Y) + (int64_t)m * p.ldy + n) = a;
            return;
        }
        float b[4], y[4];
        bias4(n, b);
        if constexpr (EPI == EPI_F32SILU) {
            const v4f u = sum4((int64_t)m * p.N + p.F + n);
            float bu[4], g[4], uu[4];
            bias4(p.F + n, bu);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                g[r] = a[r] + b[r];
                uu[r] = u[r] + bu[r];
            }
            silu_gate4(g, uu, y);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = a[r] + b[r];
        }
        *reinterpret_cast<uint2*>(Y + (int64_t)m * p.ldy + n) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
    }
}

hipError_t launch_splitk_f32_epilogue(const GemmArgs& a, int split_k, int epi, hipStream_t st) {
    Plan dummy{};
    dummy.split_k = split_k;
    KArgs k = make_kargs(a, dummy, 1);
    if (epi == EPI_F32RMSNORM) {
        const int64_t items = (int64_t)a.M * (a.N / 256);
        hipLaunchKernelGGL(splitk_f32_epi_kernel<EPI_F32RMSNORM>, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, k);
        return hipGetLastError();
    }
    const int nout = epi == EPI_F32SILU ? a.N / 2 : a.N;
    const unsigned blocks = (unsigned)(((int64_t)a.M * (nout / 4) + 255) / 256);
    switch (epi) {
        case EPI_F32BIAS: hipLaunchKernelGGL(splitk_f32_epi_kernel<EPI_F32BIAS>, dim3(blocks), dim3(256), 0, st, k); break;
        case EPI_F32SILU: hipLaunchKernelGGL(splitk_f32_epi_kernel<EPI_F32SILU>, dim3(blocks), dim3(256), 0, st, k); break;
        case EPI_ACC: hipLaunchKernelGGL(splitk_f32_epi_kernel<EPI_ACC>, dim3(blocks), dim3(256), 0, st, k); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_splitk_epilogue(const GemmArgs& a, int split_k, int epi, hipStream_t st) {
    Plan dummy{};
    dummy.split_k = split_k;
    KArgs k = make_kargs(a, dummy, 1);
    if (epi == EPI_RMSNORM) {
        const int64_t items = (int64_t)a.M * (a.N / 256);
        hipLaunchKernelGGL(splitk_epi_kernel<EPI_RMSNORM>, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, k);
        return hipGetLastError();
    }
    const int nout = epi == EPI_SILU ? a.N / 2 : a.N;
    const int64_t items = (int64_t)a.M * (nout / 4);
    const unsigned blocks = (unsigned)((items + 255) / 256);
    switch (epi) {
        case EPI_BIAS: hipLaunchKernelGGL(splitk_epi_kernel<EPI_BIAS>, dim3(blocks), dim3(256), 0, st, k); break;
        case EPI_SILU: hipLaunchKernelGGL(splitk_epi_kernel<EPI_SILU>, dim3(blocks), dim3(256), 0, st, k); break;
        case EPI_ACC: hipLaunchKernelGGL(splitk_epi_kernel<EPI_ACC>, dim3(blocks), dim3(256), 0, st, k); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qdt
