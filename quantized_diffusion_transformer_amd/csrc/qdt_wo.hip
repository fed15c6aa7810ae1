// Weight-only block-quantized linear: bf16 activations times 4-bit or 8-bit weights with a
// half-precision scale per block of 32, on the bf16 matrix cores.
//
// Method: "Quantizing a Dual-Branch Flow-Matching Diffusion Transformer for Consumer GPUs"
// (GGUF paragraph: an 8-bit round-to-nearest weight format at 8.5 bits per weight and a 4-bit
// one at 4.5 bits per weight, dequantized at run time), and "Faster Ideogram 4 with Less Prompt
// Compute", section "The NF4 Exactness Problem": the 53248-deep text projection multiplies bf16
// activations by dequantized 4-bit weights, and a kernel that changes its reduction order with
// the row count M changes the output bits, which forced that page to pad every call to the
// original 4608 rows.
//
// Design (gfx950):
//   * The dequantized weight bf16(q * d) is formed in registers right before the MFMA that reads
//     it (v_mfma_f32_16x16x32_bf16): codes and scales never pass through LDS.  One workgroup
//     of 4 waves computes a 256 x 256 tile; each wave owns 64 weight rows (4 fragments) against
//     all 256 token rows (16 fragments), so every weight element is dequantized exactly once
//     per workgroup and the token fragments are shared through LDS.
//   * The MFMA's 32 K positions are assigned so that lane group g (lanes 16 g .. 16 g + 15)
//     covers block g of each 128-element stage over the stage's 4 K steps (K step s takes
//     elements 32 g + 8 s .. + 7).  A lane then needs one contiguous block of codes (16 or 32
//     bytes, one or two global_load_dwordx4) and one scale per weight fragment and stage.  The
//     token fragments are read from LDS at the same K positions.
//   * Tokens go through LDS by LDS-DMA (256 bytes per row and stage, double buffered, rows
//     XOR-swizzled in 16-byte chunks so that one ds_read_b128 of 16 rows is conflict free).
//   * Dequantization is spread over the MFMAs: while the MFMAs of K step s run, the weight
//     fragments of step s + 1 are formed, one bf16 pair per fragment slot.
//   * Batch invariance: K is reduced in fixed slices of QDT_WO_KSLICE elements whatever M and N
//     are.  Each slice is summed by the same MFMA sequence, the slices are added in order, then
//     the bias.  An output element therefore depends only on its token row, its weight row and
//     its bias: the first T rows of a call with M rows are bit-identical to a call with T rows.
#include "qdt_device.h"
#include "qdt_internal.h"
#include "qdt_lds.h"

namespace qdt {

// ---------------------------------------------------------------------------- quantizer
// One thread per block of 32 weights: d = half(amax / qmax) (round half to even; from 65520 up
// saturated to 65504), q = clamp(rint(w / d), -qmax, qmax) with a correctly rounded fp32
// division (q = 0 when d = 0).  8-bit codes are int8; 4-bit codes are q + 8, the even element in
// the low nibble.
template <int BITS>
__global__ __launch_bounds__(256) void wo_quant_kernel(const uint16_t* __restrict__ W, int64_t ldw, int64_t N,
                                                       int64_t K, uint8_t* __restrict__ Q, uint16_t* __restrict__ D) {
    constexpr int QMAX = BITS == 8 ? 127 : 7;
    const int64_t nb = K / 32, total = N * nb;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t n = i / nb, b = i % nb;
        const v4u* src = reinterpret_cast<const v4u*>(W + n * ldw + b * 32);
        float v[32];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const v4u x = src[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[8 * c + 2 * e] = bf16_to_f32(x[e] & 0xFFFFu);
                v[8 * c + 2 * e + 1] = bf16_to_f32(x[e] >> 16);
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, __builtin_fabsf(v[j]));
        const float t = amax / (float)QMAX;
        uint16_t hb = __builtin_bit_cast(uint16_t, (_Float16)t);
        if (hb >= 0x7C00u) hb = 0x7BFFu;  // t >= 65520 rounded to infinity: saturate
        const float d = (float)__builtin_bit_cast(_Float16, hb);
        int q[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            float r = 0.0f;
            if (d > 0.0f) r = fminf(fmaxf(rintf(v[j] / d), (float)-QMAX), (float)QMAX);
            q[j] = (int)r;
        }
        D[n * nb + b] = hb;
        if constexpr (BITS == 8) {
            v4u o[2];
#pragma unroll
            for (int w = 0; w < 8; ++w)
                o[w / 4][w % 4] = (uint32_t)(q[4 * w] & 0xFF) | ((uint32_t)(q[4 * w + 1] & 0xFF) << 8) |
                                  ((uint32_t)(q[4 * w + 2] & 0xFF) << 16) | ((uint32_t)(q[4 * w + 3] & 0xFF) << 24);
            v4u* dst = reinterpret_cast<v4u*>(Q + n * K + b * 32);
            dst[0] = o[0];
            dst[1] = o[1];
        } else {
            v4u o;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t x = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) x |= (uint32_t)(q[8 * w + e] + 8) << (4 * e);
                o[w] = x;
            }
            *reinterpret_cast<v4u*>(Q + n * (K / 2) + b * 16) = o;
        }
    }
}

hipError_t launch_wo_quant(const uint16_t* W, int64_t ldw, int64_t N, int64_t K, int bits, uint8_t* Q, uint16_t* D,
                           hipStream_t st) {
    const int64_t total = N * (K / 32);
    const int64_t want = (total + 255) / 256, cap = (int64_t)kNumCU * 64;
    const unsigned blocks = (unsigned)(want < cap ? want : cap);
    if (bits == 8)
        hipLaunchKernelGGL(wo_quant_kernel<8>, dim3(blocks), dim3(256), 0, st, W, ldw, N, K, Q, D);
    else
        hipLaunchKernelGGL(wo_quant_kernel<4>, dim3(blocks), dim3(256), 0, st, W, ldw, N, K, Q, D);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- GEMM
struct WoKArgs {
    const uint16_t* X;
    int64_t ldx;
    const uint8_t* Wq;
    const uint16_t* Wd;
    const uint16_t* bias;
    void* Y;
    int64_t ldy;
    float* ws;  // fp32 partial sums [split_k][M][N] when K is split
    int M, N, K;
    int tiles_m, tiles_n, split_k, kt_total, kt_per_split;
};

// Row r mod 16 with its two 2-bit halves swapped: the token LDS swizzle.
__device__ __forceinline__ int rot4(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// MFMA with the accumulator tuple tied in place in AGPRs (see the W8A8 GEMM for why asm).
__device__ __forceinline__ void mfma_bf16_acc(v4f& c, const v4u& a, const v4u& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

template <int BITS>
struct WoRegs {
    static constexpr int NC = BITS == 8 ? 2 : 1;  // 16-byte code chunks per lane and fragment
    v4u c[4][NC];                                 // codes of the lane's block, fragments 0..3
    uint16_t s[4];                                // half-precision scale bits
};

// EPI: EPI_F32BIAS (bf16 out), EPI_ACC (fp32 accumulators out), EPI_PARTIAL (fp32 slice sums).
template <int BITS, int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void
wo_gemm_kernel(WoKArgs p) {
    constexpr int BM = 256, BN = 256, BK = 128;  // token rows, weight rows, K elements per stage
    constexpr int FM = 16, FN = 4;               // fragments per wave: token, weight
    constexpr int ROWB = BK * 2;                 // LDS bytes per token row and stage
    constexpr int STAGE = BM * ROWB;             // 64 KiB
    constexpr int NDMA = STAGE / 1024 / 4;       // LDS-DMA instructions per wave and stage
    constexpr int CB = BITS * 32 / 8;            // code bytes per block
    constexpr int SB = BK * BITS / 8;            // code bytes per weight row and stage
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---- workgroup id -> (K slice, token tile, weight tile): ids are dealt round-robin to the 8
    // XCDs, so they are remapped to give each XCD a contiguous run, in which consecutive
    // workgroups share a token tile and K slice (the token tile then stays in that XCD's L2)
    const int bid = blockIdx.x, nb = gridDim.x;
    const int xcd = bid % kNumXCD, per = nb / kNumXCD, rem = nb % kNumXCD;
    const int t = xcd * per + min(xcd, rem) + bid / kNumXCD;
    const int tn = t % p.tiles_n, tr = t / p.tiles_n;
    const int tm = tr % p.tiles_m, split = tr / p.tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int kt0 = split * p.kt_per_split;
    // stages of the slice: a multiple of 4 (K % 512 == 0, slices of 64 stages), so the main loop
    // runs stages in fours with no conditional stage (a merge of control flow would make the
    // compiler shuffle all 256 accumulator registers)
    const int nk = min(p.kt_total - kt0, p.kt_per_split);

    // ---- token LDS-DMA: instruction i of wave w fills LDS rows 4 (NDMA w + i) .. + 3 of the
    // stage (1 KiB); lane l moves row r = 4 (NDMA w + i) + l / 16 into LDS chunk slot l % 16, which
    // holds the row's global 16-byte chunk (l % 16) ^ rot4(r).  rot4 swaps the two 2-bit halves of
    // r mod 16, so each of the four 16-lane passes of a fragment read (lanes 0-3, 12-15, 20-23,
    // 24-27 and that set XORed with 4, 32, 36) lands on distinct 16-byte bank groups, which the
    // plain c ^ r does not.  Rows past M are clamped to the last row: their outputs are not stored.
    const int xlast = p.M - m0 - 1;
    const uint8_t* xbase =
        uniform_ptr(reinterpret_cast<const uint8_t*>(p.X + (int64_t)m0 * p.ldx + (int64_t)kt0 * BK));
    uint32_t xoff[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int r = 4 * (NDMA * wave + i) + (lane >> 4);
        xoff[i] = (uint32_t)((int64_t)min(r, xlast) * p.ldx * 2) + (uint32_t)(((lane & 15) ^ rot4(r)) * 16);
    }
    const uint32_t ldsx = __builtin_amdgcn_readfirstlane(lds_offset(smem) + wave * NDMA * 1024);
    auto dma_stage = [&](int buf, int j) __attribute__((always_inline)) {
        const uint8_t* sb = xbase + (int64_t)j * ROWB;
#pragma unroll
        for (int i = 0; i < NDMA; ++i) lds_dma16_s(ldsx + (uint32_t)(buf * STAGE + i * 1024), xoff[i], sb);
    };

    // ---- weight codes: lane (n = lane & 15, g = lane >> 4) of fragment f reads weight row
    // n0 + 64 wave + 16 f + n (clamped to the last row), block 4 j + g of stage j
    const int64_t qrow = BITS == 8 ? (int64_t)p.K : (int64_t)p.K / 2, srow = p.K / 32;
    const int wlast = p.N - n0 - 1;
    const uint8_t* wqbase = p.Wq + (int64_t)n0 * qrow + (int64_t)kt0 * SB;
    const uint16_t* wdbase = p.Wd + (int64_t)n0 * srow + (int64_t)kt0 * 4;
    uint32_t qoff[FN], soff[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
        const int r = min(64 * wave + 16 * f + (lane & 15), wlast);
        qoff[f] = (uint32_t)(r * qrow) + (uint32_t)((lane >> 4) * CB);
        soff[f] = (uint32_t)(r * srow) + (uint32_t)(lane >> 4);
    }
    using Regs = WoRegs<BITS>;
    auto wload = [&](Regs& R, int j) __attribute__((always_inline)) {
        const uint8_t* cb = wqbase + (int64_t)j * SB;
        const uint16_t* sp = wdbase + (int64_t)j * 4;
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int c = 0; c < Regs::NC; ++c) R.c[f][c] = *reinterpret_cast<const v4u*>(cb + qoff[f] + 16 * c);
#pragma unroll
        for (int f = 0; f < FN; ++f) R.s[f] = sp[soff[f]];
    };
    // Marks the point where a register set is first used: the compiler waits for its loads right
    // here and cannot move arithmetic on them above it (asm statements keep their order), so no
    // wait for a set lands where it would also hold back loads issued after it.  (The compiler
    // does not count the asm LDS-DMAs, so a wait it places early would cover them too.)
    auto fence = [&](Regs& R) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < FN; ++f) {
#pragma unroll
            for (int c = 0; c < Regs::NC; ++c) asm volatile("" : "+v"(R.c[f][c]));
            asm volatile("" : "+v"(R.s[f]));
        }
    };

    // ---- dequantization.  Pair p (0..3) of fragment f's 8 elements for K step s: elements
    // 2 p, 2 p + 1 of the lane's 8 (block elements 8 s + 2 p, + 1) as bf16(q * d), computed as
    // fma(code, d, -offset * d), exact in fp32 (the stored code is q + 8, or q + 128 after the
    // sign flip of the int8 byte).  Split in parts so that each can follow its own MFMA:
    // deq_src (once per fragment and step for 4 bits, per dword for 8 bits) isolates the codes as
    // bytes, deq_cvt turns two of them into floats (v_cvt_f32_ubyteN), then fma and pack.
    auto deq_src = [&](const Regs& R, int f, int s, int pr, uint32_t& lo, uint32_t& hi) __attribute__((always_inline)) {
        if constexpr (BITS == 4) {
            const uint32_t x = R.c[f][0][s];
            lo = x & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6 in bytes 0..3
            hi = (x >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
            // opaque to the optimizer, so that each element is one v_cvt_f32_ubyteN of these
            // words instead of a re-derived bit-field extract plus a conversion
            asm volatile("" : "+v"(lo), "+v"(hi));
        } else {
            const int dw = 2 * s + pr / 2;
            lo = R.c[f][dw / 4][dw % 4] ^ 0x80808080u;  // elements 4 (pr / 2) .. + 3, biased by 128
            hi = 0u;
            asm volatile("" : "+v"(lo));
        }
    };
    auto deq_cvt = [&](uint32_t lo, uint32_t hi, int pr, float& c0, float& c1) __attribute__((always_inline)) {
        if constexpr (BITS == 4) {
            c0 = (float)((lo >> (8 * pr)) & 0xFFu);
            c1 = (float)((hi >> (8 * pr)) & 0xFFu);
        } else {
            c0 = (float)((lo >> (16 * (pr & 1))) & 0xFFu);
            c1 = (float)((lo >> (16 * (pr & 1) + 8)) & 0xFFu);
        }
    };
    auto deq_pair = [&](const Regs& R, int f, int s, int pr, float d, float nod) __attribute__((always_inline)) {
        uint32_t lo, hi;
        float c0, c1;
        deq_src(R, f, s, pr, lo, hi);
        deq_cvt(lo, hi, pr, c0, c1);
        return pack_bf16x2(__builtin_fmaf(c0, d, nod), __builtin_fmaf(c1, d, nod));
    };
    constexpr float OFS = BITS == 8 ? -128.0f : -8.0f;
    auto scale_of = [&](const Regs& R, int f) __attribute__((always_inline)) {
        return (float)__builtin_bit_cast(_Float16, R.s[f]);
    };

    v4f acc[FN][FM];
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[f][fm] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // token fragment (fm, K step s) of the lane: row 16 fm + (lane & 15), chunk 4 (lane >> 4) + s
    const int frow = (lane & 15) * ROWB;
    auto tok = [&](int buf, int it) __attribute__((always_inline)) {
        const int s = it / FM, fm = it % FM;
        const int slot = ((4 * (lane >> 4) + s) ^ rot4(lane & 15)) * 16;
        return *reinterpret_cast<const v4u*>(smem + buf * STAGE + fm * 16 * ROWB + frow + slot);
    };

    // ---- one stage: wait for its LDS-DMAs and codes, publish with the barrier, start the next
    // stage's loads into the other buffers, then 4 K steps of 16 x 4 MFMAs.  The weight fragments
    // of a K step are formed during the previous one (those of step 0 during step 3 of the
    // previous stage, from the other register set, whose loads were issued a stage earlier).
    // ---- the weight codes travel in a ring of 4 register sets, loaded two stages ahead: stage j
    // computes from set j % 4 (and set (j + 1) % 4 for the next stage's step-0 fragments, during
    // its last K step) while the loads of stage j + 2 fill set (j + 2) % 4.  At the top of a stage
    // its LDS-DMAs must have landed but the NW code loads issued after them may not have:
    // vmcnt(NW).  Past the slice end, loads are clamped to its last stage (unused, in bounds),
    // which keeps the counts fixed and the loop free of branches.
    constexpr int NW = FN * Regs::NC + FN;  // VMEM instructions per wload
    Regs S0, S1, S2, S3;
    v4u a[FN];
    auto stage = [&](int j, Regs& Rc, Regs& Rn, Regs& Rl, int buf) __attribute__((always_inline)) {
        wait_vmcnt<NW>();
        fence(Rc);
        __syncthreads();
        dma_stage(buf ^ 1, min(j + 1, nk - 1));
        wload(Rl, min(j + 2, nk - 1));
        float d[FN], nod[FN], dn[FN], nodn[FN];
#pragma unroll
        for (int f = 0; f < FN; ++f) {
            d[f] = scale_of(Rc, f);
            nod[f] = d[f] * OFS;
        }
        v4u bq[3];
        bq[0] = tok(buf, 0);
        bq[1] = tok(buf, 1);
        // Each iteration: 4 MFMAs (token fragment it against the 4 weight fragments), one slice of
        // the next K step's dequantization after each MFMA (so the VALU work runs in the MFMAs'
        // shadow), and the LDS read of token fragment it + 2.
        v4u an[FN];
        uint32_t slo = 0u, shi = 0u;
#pragma unroll
        for (int it = 0; it < 4 * FM; ++it) {
            const int s = it / FM, fm = it % FM;
            const int f = fm / 4, pr = fm % 4;          // fragment and pair formed in this iteration
            const bool next = s == 3;                   // forming the next stage's step 0
            Regs& Rs = next ? Rn : Rc;
            const int ss = next ? 0 : s + 1;
            if (next && fm == 0) {
                fence(Rn);
#pragma unroll
                for (int g = 0; g < FN; ++g) {
                    dn[g] = scale_of(Rn, g);
                    nodn[g] = dn[g] * OFS;
                }
            }
            const float dd = next ? dn[f] : d[f], no = next ? nodn[f] : nod[f];
            if (fm == 0) asm volatile("s_nop 1");  // VALU-written fragments -> MFMA source
            mfma_bf16_acc(acc[0][fm], a[0], bq[it % 3]);
            if (BITS == 4 ? pr == 0 : (pr & 1) == 0) deq_src(Rs, f, ss, pr, slo, shi);
            __builtin_amdgcn_sched_barrier(0);
            mfma_bf16_acc(acc[1][fm], a[1], bq[it % 3]);
            float c0, c1;
            deq_cvt(slo, shi, pr, c0, c1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_bf16_acc(acc[2][fm], a[2], bq[it % 3]);
            const float w0 = __builtin_fmaf(c0, dd, no), w1 = __builtin_fmaf(c1, dd, no);
            __builtin_amdgcn_sched_barrier(0);
            mfma_bf16_acc(acc[3][fm], a[3], bq[it % 3]);
            an[f][pr] = pack_bf16x2(w0, w1);
            if (it + 2 < 4 * FM) bq[(it + 2) % 3] = tok(buf, it + 2);
            if (fm == FM - 1) {
#pragma unroll
                for (int g = 0; g < FN; ++g) a[g] = an[g];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // prologue: the codes of stages 0 and 1 around stage 0's LDS-DMAs (the order the stage waits
    // assume), then stage 0's step-0 weight fragments
    wload(S0, 0);
    dma_stage(0, 0);
    wload(S1, 1);
    fence(S0);
#pragma unroll
    for (int f = 0; f < FN; ++f) {
        const float d0 = scale_of(S0, f), n0d = d0 * OFS;
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) a[f][pr] = deq_pair(S0, f, 0, pr, d0, n0d);
    }
    // nk is a positive multiple of 4 (K % 512 == 0).  The loop leaves only through the drain, so
    // the register copies the compiler places on its exit edge read finished accumulators.
    for (int j = 0;; j += 4) {
        stage(j, S0, S1, S2, 0);
        stage(j + 1, S1, S2, S3, 1);
        stage(j + 2, S2, S3, S0, 0);
        stage(j + 3, S3, S0, S1, 1);
        if (j + 4 >= nk) {
            mfma_drain();
            break;
        }
    }
    wait_vmcnt<0>();  // the clamped LDS-DMAs of the last stage land before the workgroup ends
    mfma_drain();
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) keep_after_a(acc[f][fm]);

    // ---------------------------------------------------------------- epilogue
    // Lane l of fragment (f, fm) holds outputs of token row m0 + 16 fm + (l & 15) and weight rows
    // (output columns) n0 + 64 wave + 16 f + 4 (l >> 4) .. + 3.
    const int ncol = n0 + 64 * wave + 4 * (lane >> 4);
    float b[FN][4];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
        const int n = ncol + 16 * f;
#pragma unroll
        for (int r = 0; r < 4; ++r) b[f][r] = 0.0f;
        if constexpr (EPI == EPI_F32BIAS) {
            if (p.bias && n < p.N) {
                const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
                b[f][0] = bf16_to_f32(bb.x & 0xFFFFu);
                b[f][1] = bf16_to_f32(bb.x >> 16);
                b[f][2] = bf16_to_f32(bb.y & 0xFFFFu);
                b[f][3] = bf16_to_f32(bb.y >> 16);
            }
        }
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + 16 * fm + (lane & 15);
        if (m >= p.M) continue;
#pragma unroll
        for (int f = 0; f < FN; ++f) {
            const int n = ncol + 16 * f;
            if (n >= p.N) continue;
            const v4f v = acc[f][fm];
            if constexpr (EPI == EPI_F32BIAS) {
                uint16_t* Y = reinterpret_cast<uint16_t*>(p.Y) + (int64_t)m * p.ldy + n;
                const uint2 o = make_uint2(pack_bf16x2(v[0] + b[f][0], v[1] + b[f][1]),
                                           pack_bf16x2(v[2] + b[f][2], v[3] + b[f][3]));
                __builtin_nontemporal_store(o.x, reinterpret_cast<uint32_t*>(Y));
                __builtin_nontemporal_store(o.y, reinterpret_cast<uint32_t*>(Y) + 1);
            } else if constexpr (EPI == EPI_ACC) {
                *reinterpret_cast<v4f*>(reinterpret_cast<float*>(p.Y) + (int64_t)m * p.ldy + n) = v;
            } else {
                *reinterpret_cast<v4f*>(p.ws + ((int64_t)split * p.M + m) * p.N + n) = v;
            }
        }
    }
}

hipError_t launch_wo_gemm(const uint16_t* X, int64_t ldx, const uint8_t* Wq, const uint16_t* Wd, int bits,
                          const uint16_t* bias, int M, int N, int K, int epi, void* Y, int64_t ldy, float* ws,
                          const Plan& pl, hipStream_t st) {
    WoKArgs k;
    k.X = X;
    k.ldx = ldx;
    k.Wq = Wq;
    k.Wd = Wd;
    k.bias = bias;
    k.Y = Y;
    k.ldy = ldy;
    k.ws = ws;
    k.M = M;
    k.N = N;
    k.K = K;
    k.tiles_m = pl.tiles_m;
    k.tiles_n = pl.tiles_n;
    k.split_k = pl.split_k;
    k.kt_total = pl.kt_total;
    k.kt_per_split = pl.kt_per_split;
    const int e = pl.split_k > 1 ? EPI_PARTIAL : epi;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(256), 0, st, k);
        return hipGetLastError();
    };
    if (bits == 8) {
        if (e == EPI_PARTIAL) return go(wo_gemm_kernel<8, EPI_PARTIAL>);
        if (e == EPI_ACC) return go(wo_gemm_kernel<8, EPI_ACC>);
        return go(wo_gemm_kernel<8, EPI_F32BIAS>);
    }
    if (e == EPI_PARTIAL) return go(wo_gemm_kernel<4, EPI_PARTIAL>);
    if (e == EPI_ACC) return go(wo_gemm_kernel<4, EPI_ACC>);
    return go(wo_gemm_kernel<4, EPI_F32BIAS>);
}

}  // namespace qdt
