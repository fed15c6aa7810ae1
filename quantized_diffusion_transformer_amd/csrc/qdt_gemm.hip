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
//   * One workgroup of 4 waves (one per SIMD) computes a BM x BN tile; each wave owns an
//     (FM*16) x (FN*16) sub-tile as FN x FM accumulators of v_mfma_i32_16x16x64_i8
//     (v_mfma_f32_16x16x32_bf16 for bf16).  The MFMA A operand is the weight fragment and
//     the B operand the token fragment, so lane l holds 4 consecutive output columns of one
//     output row: the epilogue stores 8 bytes per lane straight from registers.
//   * K advances 128 bytes per stage.  Global -> VGPR prefetch of stage k+1 overlaps the
//     MFMAs of stage k; LDS is double buffered (one barrier per stage).  Rows are 128 bytes
//     in LDS with the 16-byte chunks XOR-swizzled by (row & 7) so that the 16 rows read by
//     one ds_read_b128 fall in distinct banks.
//   * Tile order is XCD-aware: workgroup ids are dealt round-robin to the 8 XCDs, so ids are
//     remapped to give each XCD a contiguous run of tiles, walked in groups of `group_m` tile
//     rows, which keeps the operands of neighbouring tiles in that XCD's L2.
//   * Rows beyond M (or N) load zeros and are not stored; the integer sum is exact, so the
//     result is independent of the tile shape and of the K split.
#include "qdt_device.h"
#include "qdt_internal.h"

namespace qdt {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct KArgs {
    const uint8_t* X;
    const uint8_t* W;
    const float* sx;
    const float* sw;
    const uint16_t* bias;
    const uint16_t* gamma;
    void* Y;
    int32_t* ws;
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

template <bool BF16>
__device__ __forceinline__ typename AccT<BF16>::type mfma(const uint4& a, const uint4& b, typename AccT<BF16>::type c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                      0);
    } else {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, a), __builtin_bit_cast(v4i, b), c, 0, 0, 0);
    }
}

// WM x WN waves, FM x FN fragments of 16x16 per wave.  PHASED: prefetch the weight half of
// the next stage before the first K sub-step and the token half before the second one
// (halves the prefetch registers of the large tile).
template <int WM, int WN, int FM, int FN, bool BF16, int EPI, bool PHASED>
__global__ __attribute__((amdgpu_flat_work_group_size(WM * WN * 64, WM * WN * 64), amdgpu_waves_per_eu(1, 1))) void
gemm_kernel(KArgs p) {
    constexpr int NT = WM * WN * 64;
    constexpr int BM = WM * FM * 16;
    constexpr int BN = WN * FN * 16;
    constexpr int BKC = 8;  // 16-byte chunks per row per stage
    constexpr int BK = BKC * 16;
    constexpr int ROWS = BN + BM;  // LDS rows per stage: weight rows, then token rows
    constexpr int STAGE = ROWS * BK;
    constexpr int RSTEP = NT / BKC;
    constexpr int CW = BN / RSTEP, CX = BM / RSTEP;
    constexpr bool SILU = EPI == EPI_SILU;
    static_assert(BN % RSTEP == 0 && BM % RSTEP == 0, "tile rows must be a multiple of the load row step");
    static_assert(!SILU || ((BN / 2) % RSTEP == 0 && FN % 2 == 0), "gate/up halves must align");
    using Acc = typename AccT<BF16>::type;

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
    __shared__ float red[EPI == EPI_RMSNORM ? WN * BM : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % WN, wm = wave / WN;

    // ---- workgroup id -> (tile, K slice), contiguous per XCD
    const int bid = blockIdx.x, nb = gridDim.x;
    const int xcd = bid % kNumXCD, per = nb / kNumXCD, rem = nb % kNumXCD;
    const int t = xcd * per + min(xcd, rem) + bid / kNumXCD;
    const int split = t % p.split_k;
    const int tt = t / p.split_k;
    const int gsz = p.group_m * p.tiles_n;
    const int first_m = (tt / gsz) * p.group_m;
    const int gm = min(p.tiles_m - first_m, p.group_m);
    const int tm = first_m + (tt % gsz) % gm;
    const int tn = (tt % gsz) / gm;
    const int m0 = tm * BM;
    const int n0 = tn * (SILU ? BN / 2 : BN);  // first output column (SILU) / weight row
    const int kt0 = split * p.kt_per_split;
    const int kt1 = min(p.kt_total, kt0 + p.kt_per_split);

    // ---- global load assignment: chunk kc of rows rb + i * RSTEP
    const int kc = tid % BKC, rb = tid / BKC;
    const int64_t Kb = p.Kb;
    const int nlim = SILU ? p.F : p.N;
    const uint8_t* pw = p.W + (int64_t)(n0 + rb) * Kb + kc * 16;
    const uint8_t* pwu = SILU ? p.W + (int64_t)(p.F + n0 + rb) * Kb + kc * 16 : pw;
    const uint8_t* px = p.X + (int64_t)(m0 + rb) * Kb + kc * 16;
    const int w_rows_left = nlim - n0 - rb;  // chunk i valid iff i * RSTEP < rows_left
    const int x_rows_left = p.M - m0 - rb;
    const int64_t rstride = (int64_t)RSTEP * Kb;
    const int st_off = rb * BK + ((kc ^ (rb & 7)) << 4);  // swizzled LDS offset of this thread's chunk

    uint4 rw[CW], rx[CX];
    auto load_w = [&](int kt) {
        const int64_t ko = (int64_t)kt * BK;
        const bool kok = ko + kc * 16 < Kb;
#pragma unroll
        for (int i = 0; i < CW; ++i) {
            const int ii = SILU && i >= CW / 2 ? i - CW / 2 : i;
            const uint8_t* base = SILU && i >= CW / 2 ? pwu : pw;
            if (kok && ii * RSTEP < w_rows_left)
                rw[i] = *reinterpret_cast<const uint4*>(base + ii * rstride + ko);
            else
                rw[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto load_x = [&](int kt) {
        const int64_t ko = (int64_t)kt * BK;
        const bool kok = ko + kc * 16 < Kb;
#pragma unroll
        for (int i = 0; i < CX; ++i) {
            if (kok && i * RSTEP < x_rows_left)
                rx[i] = *reinterpret_cast<const uint4*>(px + i * rstride + ko);
            else
                rx[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_w = [&](int buf) {
        uint8_t* s = smem + buf * STAGE + st_off;
#pragma unroll
        for (int i = 0; i < CW; ++i) *reinterpret_cast<uint4*>(s + i * RSTEP * BK) = rw[i];
    };
    auto store_x = [&](int buf) {
        uint8_t* s = smem + buf * STAGE + BN * BK + st_off;
#pragma unroll
        for (int i = 0; i < CX; ++i) *reinterpret_cast<uint4*>(s + i * RSTEP * BK) = rx[i];
    };

    // ---- fragment read offsets: row (lane & 15) of a 16-row fragment, chunk 4*ks + (lane >> 4)
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
    const int lck0 = (((lane >> 4) + 0) ^ (lane & 7)) << 4;
    const int lck1 = (((lane >> 4) + 4) ^ (lane & 7)) << 4;

    Acc acc[FN][FM];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = Acc{0, 0, 0, 0};

    auto compute = [&](int buf, int ks) {
        const uint8_t* s = smem + buf * STAGE + lrow + (ks ? lck1 : lck0);
        uint4 a[FN], b[FM];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) a[fn] = *reinterpret_cast<const uint4*>(s + wrow[fn] * BK);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) b[fm] = *reinterpret_cast<const uint4*>(s + (xrow0 + fm * 16) * BK);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = mfma<BF16>(a[fn], b[fm], acc[fn][fm]);
    };

    if (kt0 < kt1) {
        load_w(kt0);
        load_x(kt0);
        store_w(0);
        store_x(0);
        __syncthreads();
        for (int kt = kt0; kt < kt1; ++kt) {
            const int cur = (kt - kt0) & 1;
            const bool more = kt + 1 < kt1;
            if (more) {
                load_w(kt + 1);
                if constexpr (!PHASED) load_x(kt + 1);
            }
            compute(cur, 0);
            if (more) {
                store_w(cur ^ 1);
                if constexpr (PHASED) load_x(kt + 1);
            }
            compute(cur, 1);
            if (more) store_x(cur ^ 1);
            __syncthreads();
        }
    }

    // ---------------------------------------------------------------- epilogues
    const int mrow0 = m0 + wm * FM * 16 + (lane & 15);  // + fm * 16
    const int ncol0 = wn * (SILU ? FN / 2 : FN) * 16 + 4 * (lane >> 4);  // + n0 + fn * 16

    if constexpr (EPI == EPI_ACC || EPI == EPI_PARTIAL) {
        int32_t* out = EPI == EPI_ACC ? reinterpret_cast<int32_t*>(p.Y) : p.ws + (int64_t)split * p.M * p.N;
        const int64_t ld = EPI == EPI_ACC ? p.ldy : p.N;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = n0 + ncol0 + fn * 16;
            if (n >= p.N) continue;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int m = mrow0 + fm * 16;
                if (m < p.M) *reinterpret_cast<v4i*>(out + (int64_t)m * ld + n) = acc[fn][fm];
            }
        }
    } else if constexpr (EPI == EPI_F32BIAS) {
        uint16_t* Y = reinterpret_cast<uint16_t*>(p.Y);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = n0 + ncol0 + fn * 16;
            if (n >= p.N) continue;
            float b[4] = {0.f, 0.f, 0.f, 0.f};
            if (p.bias) {
                uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
                b[0] = bf16_to_f32(bb.x & 0xFFFFu); b[1] = bf16_to_f32(bb.x >> 16);
                b[2] = bf16_to_f32(bb.y & 0xFFFFu); b[3] = bf16_to_f32(bb.y >> 16);
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int m = mrow0 + fm * 16;
                if (m >= p.M) continue;
                float y[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) y[r] = p.bias ? (float)acc[fn][fm][r] + b[r] : (float)acc[fn][fm][r];
                *reinterpret_cast<uint2*>(Y + (int64_t)m * p.ldy + n) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
            }
        }
    } else if constexpr (EPI == EPI_BIAS) {
        uint16_t* Y = reinterpret_cast<uint16_t*>(p.Y);
        float sxv[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) sxv[fm] = mrow0 + fm * 16 < p.M ? p.sx[mrow0 + fm * 16] : 0.0f;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = n0 + ncol0 + fn * 16;
            if (n >= p.N) continue;
            const float4 sw = *reinterpret_cast<const float4*>(p.sw + n);
            float b[4] = {0.f, 0.f, 0.f, 0.f};
            if (p.bias) {
                uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
                b[0] = bf16_to_f32(bb.x & 0xFFFFu); b[1] = bf16_to_f32(bb.x >> 16);
                b[2] = bf16_to_f32(bb.y & 0xFFFFu); b[3] = bf16_to_f32(bb.y >> 16);
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int m = mrow0 + fm * 16;
                if (m >= p.M) continue;
                const float y0 = dequant(acc[fn][fm][0], sxv[fm], sw.x, b[0]);
                const float y1 = dequant(acc[fn][fm][1], sxv[fm], sw.y, b[1]);
                const float y2 = dequant(acc[fn][fm][2], sxv[fm], sw.z, b[2]);
                const float y3 = dequant(acc[fn][fm][3], sxv[fm], sw.w, b[3]);
                *reinterpret_cast<uint2*>(Y + (int64_t)m * p.ldy + n) = make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
            }
        }
    } else if constexpr (EPI == EPI_SILU) {
        uint16_t* Y = reinterpret_cast<uint16_t*>(p.Y);
        float sxv[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) sxv[fm] = mrow0 + fm * 16 < p.M ? p.sx[mrow0 + fm * 16] : 0.0f;
#pragma unroll
        for (int fn = 0; fn < FN / 2; ++fn) {
            const int f = n0 + ncol0 + fn * 16;
            if (f >= p.F) continue;
            const float4 swg = *reinterpret_cast<const float4*>(p.sw + f);
            const float4 swu = *reinterpret_cast<const float4*>(p.sw + p.F + f);
            float bg[4] = {0.f, 0.f, 0.f, 0.f}, bu[4] = {0.f, 0.f, 0.f, 0.f};
            if (p.bias) {
                uint2 g2 = *reinterpret_cast<const uint2*>(p.bias + f);
                uint2 u2 = *reinterpret_cast<const uint2*>(p.bias + p.F + f);
                bg[0] = bf16_to_f32(g2.x & 0xFFFFu); bg[1] = bf16_to_f32(g2.x >> 16);
                bg[2] = bf16_to_f32(g2.y & 0xFFFFu); bg[3] = bf16_to_f32(g2.y >> 16);
                bu[0] = bf16_to_f32(u2.x & 0xFFFFu); bu[1] = bf16_to_f32(u2.x >> 16);
                bu[2] = bf16_to_f32(u2.y & 0xFFFFu); bu[3] = bf16_to_f32(u2.y >> 16);
            }
            const float swgv[4] = {swg.x, swg.y, swg.z, swg.w};
            const float swuv[4] = {swu.x, swu.y, swu.z, swu.w};
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int m = mrow0 + fm * 16;
                if (m >= p.M) continue;
                float y[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float g = dequant(acc[fn][fm][r], sxv[fm], swgv[r], bg[r]);
                    const float u = dequant(acc[fn + FN / 2][fm][r], sxv[fm], swuv[r], bu[r]);
                    y[r] = silu_gate(g, u);
                }
                *reinterpret_cast<uint2*>(Y + (int64_t)m * p.ldy + f) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
            }
        }
    } else if constexpr (EPI == EPI_RMSNORM) {
        // The workgroup's BN = 256 columns are exactly one head; each wave holds FN*16 of
        // them, so a head spans the fragments of WN waves.  Row sums of y^2: in-lane over
        // fragments, across the 4 lane groups with shuffles, across waves through LDS, in a
        // fixed order.
        static_assert(BN == 256, "one head per tile");
        uint16_t* Y = reinterpret_cast<uint16_t*>(p.Y);
        float sxv[FM], ss[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            sxv[fm] = mrow0 + fm * 16 < p.M ? p.sx[mrow0 + fm * 16] : 0.0f;
            ss[fm] = 0.0f;
        }
        float swv[FN][4], bv[FN][4];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = n0 + ncol0 + fn * 16;
            const float4 sw = *reinterpret_cast<const float4*>(p.sw + n);
            swv[fn][0] = sw.x; swv[fn][1] = sw.y; swv[fn][2] = sw.z; swv[fn][3] = sw.w;
            if (p.bias) {
                uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
                bv[fn][0] = bf16_to_f32(bb.x & 0xFFFFu); bv[fn][1] = bf16_to_f32(bb.x >> 16);
                bv[fn][2] = bf16_to_f32(bb.y & 0xFFFFu); bv[fn][3] = bf16_to_f32(bb.y >> 16);
            } else {
                bv[fn][0] = bv[fn][1] = bv[fn][2] = bv[fn][3] = 0.0f;
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float y = dequant(acc[fn][fm][r], sxv[fm], swv[fn][r], bv[fn][r]);
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
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int d = ncol0 + fn * 16;  // column within the head
            const int n = n0 + d;
            uint2 gg = *reinterpret_cast<const uint2*>(p.gamma + d);
            const float g[4] = {bf16_to_f32(gg.x & 0xFFFFu), bf16_to_f32(gg.x >> 16), bf16_to_f32(gg.y & 0xFFFFu),
                                bf16_to_f32(gg.y >> 16)};
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int m = mrow0 + fm * 16;
                if (m >= p.M) continue;
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float y = dequant(acc[fn][fm][r], sxv[fm], swv[fn][r], bv[fn][r]);
                    o[r] = (y * rinv[fm]) * g[r];
                }
                *reinterpret_cast<uint2*>(Y + (int64_t)m * p.ldy + n) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            }
        }
    }
}

// ---------------------------------------------------------------------------- split-K epilogue
// Sums the S int32 partial slices (exact, any order) and applies the same epilogue
// arithmetic as the fused kernel.  BIAS / SILU / ACC: one thread per 4 output columns.
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
        float y[4], ss = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            y[r] = dequant(a[r], sx, swv[r], b[r]);
            ss += y[r] * y[r];
        }
        ss = wave_sum(ss);
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
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = silu_gate(dequant(a[r], sx, swv[r], b[r]), dequant(u[r], sx, swuv[r], bu[r]));
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
    return k;
}

template <int FMN, bool BF16, int EPI, bool PHASED>
static hipError_t go(const KArgs& k, int grid, hipStream_t st) {
    hipLaunchKernelGGL((gemm_kernel<2, 2, FMN, FMN, BF16, EPI, PHASED>), dim3(grid), dim3(256), 0, st, k);
    return hipGetLastError();
}

hipError_t launch_gemm_i8(const GemmArgs& a, const Plan& pl, hipStream_t st) {
    KArgs k = make_kargs(a, pl, 1);
    const int epi = pl.split_k > 1 ? EPI_PARTIAL : a.epi;
    if (pl.tile == QDT_TILE_288) {
        switch (epi) {
            case EPI_BIAS: return go<9, false, EPI_BIAS, true>(k, pl.grid, st);
            case EPI_ACC: return go<9, false, EPI_ACC, true>(k, pl.grid, st);
            case EPI_PARTIAL: return go<9, false, EPI_PARTIAL, true>(k, pl.grid, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (epi) {
        case EPI_BIAS: return go<8, false, EPI_BIAS, false>(k, pl.grid, st);
        case EPI_SILU: return go<8, false, EPI_SILU, false>(k, pl.grid, st);
        case EPI_RMSNORM: return go<8, false, EPI_RMSNORM, false>(k, pl.grid, st);
        case EPI_ACC: return go<8, false, EPI_ACC, false>(k, pl.grid, st);
        case EPI_PARTIAL: return go<8, false, EPI_PARTIAL, false>(k, pl.grid, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_bf16(const GemmArgs& a, const Plan& pl, hipStream_t st) {
    KArgs k = make_kargs(a, pl, 2);
    if (pl.tile == QDT_TILE_288) return go<9, true, EPI_F32BIAS, true>(k, pl.grid, st);
    return go<8, true, EPI_F32BIAS, false>(k, pl.grid, st);
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
