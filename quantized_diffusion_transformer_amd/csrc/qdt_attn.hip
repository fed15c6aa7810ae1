// Softmax attention per 256-wide head, after the QK-norm projection.
//
// Method: "Serving sub-second Ideogram v4 without quality loss" (the DiT's attention heads are 256
// wide; the attention runs over the joint sequence of text and image tokens).  Per head h:
// O = softmax(Q K^T / 16) V over all S tokens (no mask; 1/16 = 1/sqrt(256)).  Q, K, V and O are
// token-major [S, ld] with head h in columns 256 h .. 256 h + 255, as the projections write them.
//
// Design (gfx950):
//   * One workgroup of 4 waves takes 256 queries of one head; each wave holds 64 queries' Q in
//     registers (the B operand of the score MFMAs) and their 64 x 256 output accumulators in the
//     256 AGPRs.  Keys stream through LDS in tiles of 32 (K rows and the matching V^T rows, double
//     buffered by LDS-DMA), so each K or V element read from LDS feeds 64 queries' MFMAs.
//   * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16): a lane then holds
//     8 keys of one query per 16-query fragment, so the row max and the row sum are mostly
//     lane-local (two cross-lane steps for the max, one reduction at the very end for the sum).
//     The probabilities come out of that MFMA already in the B-operand layout of O^T += V^T P^T
//     when V^T stores each 32-key group in the order [4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3]
//     for lane group g = 0..3: the transpose pre-pass writes V^T that way.
//   * Softmax in base 2 against a fixed per-query reference: the max of the first key tile.  The
//     accumulators are never rescaled (rescaling the 256 AGPR accumulators inside the loop costs
//     more VALU than the MFMAs it feeds, and any conditional update of them makes the compiler
//     spill the query registers).  Later keys may exceed the reference: their probabilities are
//     2^((s - m) C) > 1, which bf16 (fp32's exponent range) and the fp32 sums hold up to 2^64.  A
//     workgroup in which some lane's partial row sum passes 2^64 (as it does whenever a score
//     passes the reference by more than 64 in log2 units) raises a flag; a second launch of the
//     kernel (EXACT) recomputes exactly those workgroups with the exact row max from a first pass
//     over the keys, and returns at once everywhere else.
//   * Probabilities enter the second MFMA as bf16 (as in every bf16 flash-attention kernel); the
//     row sums use the fp32 values.
#include "qdt_device.h"
#include "qdt_internal.h"
#include "qdt_lds.h"

namespace qdt {

constexpr int AT_D = 256;   // head width
constexpr int AT_BQ = 256;  // queries per workgroup (64 per wave)
constexpr int AT_BK = 32;   // keys per tile
constexpr int AT_LA = 4;    // LDS fragment reads in flight ahead of the MFMA group that uses them

// Key (0..31) stored at position p of a 32-key group of V^T.
__device__ __forceinline__ int vt_key_of_pos(int p) {
    return 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3);
}

// ---------------------------------------------------------------------------- V -> V^T
// Block (64-key block kb, head h): V rows kb*64 .. +63 of head h into LDS, then each thread writes
// one dim row of V^T: 64 keys in the permuted order, zeros past S.
__global__ __launch_bounds__(256) void attn_vt_kernel(const uint16_t* __restrict__ V, int64_t ld, int S, int Spad,
                                                      uint16_t* __restrict__ Vt, int* __restrict__ redo, int nredo) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][AT_D];
    const int kb = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    if (kb == 0 && h == 0)
        for (int i = tid; i < nredo; i += 256) redo[i] = 0;
    const int k0 = kb * 64;
    for (int c = tid; c < 64 * (AT_D / 8); c += 256) {
        const int r = c / (AT_D / 8), ch = c % (AT_D / 8);
        const int key = k0 + r;
        v4u v = {0u, 0u, 0u, 0u};
        if (key < S) v = *reinterpret_cast<const v4u*>(V + (int64_t)key * ld + h * AT_D + ch * 8);
        *reinterpret_cast<v4u*>(&tile[r][ch * 8]) = v;
    }
    __syncthreads();
    const int d = tid;
    uint16_t* dst = Vt + ((int64_t)h * AT_D + d) * Spad + k0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int grp = q / 4;
        if (k0 + 32 * grp >= Spad) break;
        v4u o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int p0 = (q % 4) * 8 + 2 * e;
            const uint32_t lo = tile[32 * grp + vt_key_of_pos(p0)][d];
            const uint32_t hi = tile[32 * grp + vt_key_of_pos(p0 + 1)][d];
            o[e] = lo | (hi << 16);
        }
        *reinterpret_cast<v4u*>(dst + q * 8) = o;
    }
}

// ---------------------------------------------------------------------------- attention
struct AttnArgs {
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* Vt;
    uint16_t* O;
    int* redo;  // per workgroup: scores outgrew the reference (cleared by the V^T pass)
    int64_t ld, ldo;
    int S, Spad, H, tiles_q;
};

// Output MFMA with the accumulator tuple tied in place in AGPRs (all 256 AGPRs hold accumulators).
__device__ __forceinline__ void mfma_o(v4f& c, const v4u& a, const v4u& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// Score MFMA with its accumulator in VGPRs (the softmax reads it; the AGPRs are all taken by the
// output).  Asm, so the kernel drains the MFMA pipeline itself before the scores are read.
__device__ __forceinline__ void mfma_s(v4f& c, const v4u& a, const v4u& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// The same with a zero accumulator (inline constant 0), for the first K step of a fragment.
__device__ __forceinline__ void mfma_s0(v4f& c, const v4u& a, const v4u& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
// LDS swizzles.  A fragment read touches 16 rows x 4 chunks of 16 bytes (64 lanes, 1 KiB).  The LDS
// (64 banks of 4 bytes) serves a 16-byte read in four passes of 16 lanes: lanes 0-3, 12-15, 20-23
// and 24-27 form one pass, the other passes are the same set XORed with 4, 32 and 36.  The slot
// permutations below put each pass on 16 distinct 16-byte bank groups.
// K rows (512 bytes, 32 chunks): chunk c of row r in slot c ^ (r mod 16).
__device__ __forceinline__ int at_ksw(int n) { return n & 15; }
// V^T rows (64 bytes, 4 chunks): chunk c of row r in slot c ^ (bit 3 of r, moved to bit 1).
__device__ __forceinline__ int at_vsw(int r) { return (r >> 2) & 2; }

template <bool EXACT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void
attn_fwd_kernel(AttnArgs p) {
    constexpr int KROW = AT_D * 2;           // LDS bytes per key row
    constexpr int KT = AT_BK * KROW;         // 16 KiB K tile
    constexpr int VROW = AT_BK * 2;          // LDS bytes per V^T dim row
    constexpr int VT = AT_D * VROW;          // 16 KiB V^T tile
    constexpr int STG = KT + VT;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STG];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bid = blockIdx.x, nb = gridDim.x;
    const int xcd = bid % kNumXCD, per = nb / kNumXCD, rem = nb % kNumXCD;
    const int t = xcd * per + min(xcd, rem) + bid / kNumXCD;  // contiguous per XCD: one head's tiles
    const int h = t / p.tiles_q, qt = t % p.tiles_q;
    const int q0 = qt * AT_BQ + 64 * wave;  // the wave's first query
    const int nkt = p.Spad / AT_BK;
    if constexpr (EXACT) {
        if (__builtin_amdgcn_readfirstlane(p.redo[t]) == 0) return;
    }

    // ---- Q fragments (B operand of S^T = K Q^T): lane holds query 16 qf + (lane & 15) of the wave,
    // dims 32 kk + 8 (lane >> 4) .. + 7.  Queries past S are clamped (their outputs are not stored).
    v4u qfr[4][8];
#pragma unroll
    for (int qf = 0; qf < 4; ++qf) {
        const int qr = min(q0 + 16 * qf + (lane & 15), p.S - 1);
        const uint16_t* src = p.Q + (int64_t)qr * p.ld + h * AT_D + 8 * (lane >> 4);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qfr[qf][kk] = *reinterpret_cast<const v4u*>(src + 32 * kk);
    }
    // the compiler's wait for these loads belongs here, before the first LDS-DMA: placed at their
    // first use inside the loop it would also hold back every tile's prefetch (the asm LDS-DMAs
    // count in the same load counter)
#pragma unroll
    for (int qf = 0; qf < 4; ++qf)
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) asm volatile("" : "+v"(qfr[qf][kk]));

    // ---- LDS-DMA of a tile: 16 instructions for K (2 key rows each), 16 for V^T (16 dim rows of
    // 64 bytes each); wave w issues 4 of each, each lane moving the global chunk that belongs in
    // its LDS slot under the swizzles above.  Keys past S are clamped to the last key (their
    // scores are masked).
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.K + h * AT_D);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.Vt + (int64_t)h * AT_D * p.Spad);
    const uint32_t ldsk = __builtin_amdgcn_readfirstlane(lds_offset(smem) + wave * 4 * 1024);
    const uint32_t ldsv = ldsk + KT;
    // Per-lane offsets, computed once: K instruction i of this wave moves key rows
    // 2 (4 w + i) + (lane >> 5) of the tile, V^T instruction i dim rows 16 (4 w + i) + lane / 4
    // (the i-dependence of the V^T offset is uniform and goes into the scalar base).  Only a
    // partial last key tile recomputes its K offsets, with rows past S clamped to the last key
    // (their scores are masked).
    uint32_t koff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 2 * (4 * wave + i) + (lane >> 5);
        koff[i] = (uint32_t)(row * p.ld * 2) + (uint32_t)(((lane & 31) ^ at_ksw(row & 15)) * 16);
    }
    const uint32_t voff = (uint32_t)((64 * wave + (lane >> 2)) * p.Spad * 2) +
                          (uint32_t)(((lane & 3) ^ at_vsw(lane >> 2)) * 16);
    auto dma_k = [&](int buf, int jt, int i) __attribute__((always_inline)) {
        const int key0 = jt * AT_BK;
        uint32_t off = koff[i];
        if (key0 + AT_BK > p.S) {
            const int row = 2 * (4 * wave + i) + (lane >> 5);
            off = (uint32_t)(min(row, p.S - 1 - key0) * p.ld * 2) + (uint32_t)(((lane & 31) ^ at_ksw(row & 15)) * 16);
        }
        lds_dma16_s(ldsk + (uint32_t)(buf * STG + i * 1024), off, kbase + (int64_t)key0 * p.ld * 2);
    };
    auto dma_v = [&](int buf, int jt, int i) __attribute__((always_inline)) {
        lds_dma16_s(ldsv + (uint32_t)(buf * STG + i * 1024), voff,
                    vbase + (int64_t)jt * AT_BK * 2 + (int64_t)16 * i * p.Spad * 2);
    };
    // K fragment (A operand): key 16 kf + (lane & 15) of the tile, dims 32 kk + 8 (lane >> 4) .. + 7
    auto kfrag = [&](int buf, int kf, int kk) __attribute__((always_inline)) {
        const int row = 16 * kf + (lane & 15);
        const int slot = (4 * kk + (lane >> 4)) ^ at_ksw(lane & 15);
        return *reinterpret_cast<const v4u*>(smem + buf * STG + row * KROW + slot * 16);
    };
    // V^T fragment (A operand): dim 16 df + (lane & 15), tile positions 8 (lane >> 4) .. + 7
    auto vfrag = [&](int buf, int df) __attribute__((always_inline)) {
        const int row = 16 * df + (lane & 15);
        return *reinterpret_cast<const v4u*>(smem + buf * STG + KT + row * VROW +
                                             (((lane >> 4) ^ at_vsw(lane & 15)) * 16));
    };

    // ---- scores of the key tile in K buffer buf: S^T = K Q^T, lane holds keys
    // 16 kf + 4 (lane >> 4) + r of query 16 qf + (lane & 15).  hook(g) runs after MFMA group g
    // (0..15): the next tiles' LDS-DMAs go there, between the MFMAs.
    v4f s[2][4];
    // drain: wait for the last MFMAs' results here (needed when VALU reads or writes the scores
    // at once); in the main loop the first such read comes at least five MFMAs later.
    auto scores = [&](int buf, auto&& hook, bool drain) __attribute__((always_inline)) {
        // 16 K fragments, each read AT_LA groups of 4 MFMAs ahead of its use (one group, 64 MFMA
        // cycles, is shorter than the LDS read latency)
        v4u a[16];
#pragma unroll
        for (int g = 0; g < AT_LA; ++g) a[g] = kfrag(buf, g / 8, g % 8);
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            if (g + AT_LA < 16) a[g + AT_LA] = kfrag(buf, (g + AT_LA) / 8, (g + AT_LA) % 8);
#pragma unroll
            for (int qf = 0; qf < 4; ++qf) {
                if (g % 8 == 0)
                    mfma_s0(s[g / 8][qf], a[g], qfr[qf][0]);
                else
                    mfma_s(s[g / 8][qf], a[g], qfr[qf][g % 8]);
            }
            hook(g);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (drain) {
            mfma_drain();
#pragma unroll
            for (int kf = 0; kf < 2; ++kf)
#pragma unroll
                for (int qf = 0; qf < 4; ++qf) keep_after_v(s[kf][qf]);
        }
    };
    // keys past S get -inf
    auto mask_tail = [&](int jt) __attribute__((always_inline)) {
        if ((jt + 1) * AT_BK > p.S) {
            mfma_drain();
#pragma unroll
            for (int kf = 0; kf < 2; ++kf)
#pragma unroll
                for (int qf = 0; qf < 4; ++qf) keep_after_v(s[kf][qf]);
#pragma unroll
            for (int kf = 0; kf < 2; ++kf)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool out = jt * AT_BK + 16 * kf + 4 * (lane >> 4) + r >= p.S;
#pragma unroll
                    for (int qf = 0; qf < 4; ++qf)
                        if (out) s[kf][qf][r] = -__builtin_inff();
                }
        }
    };
    // the tile's max per query (all lane groups), raw score units
    auto tile_max = [&](int qf) __attribute__((always_inline)) {
        float m = fmaxf(fmaxf(fmaxf(s[0][qf][0], s[0][qf][1]), fmaxf(s[0][qf][2], s[0][qf][3])),
                        fmaxf(fmaxf(s[1][qf][0], s[1][qf][1]), fmaxf(s[1][qf][2], s[1][qf][3])));
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        return fmaxf(m, __shfl_xor(m, 32, 64));
    };
    constexpr float C = 1.44269504088896341f / 16.0f;  // log2(e) / sqrt(256)

    // reference max per query fragment (raw score units) and this lane's partial row sums
    float mu[4], lp[4];
#pragma unroll
    for (int qf = 0; qf < 4; ++qf) {
        mu[qf] = -__builtin_inff();
        lp[qf] = 0.0f;
    }
    if constexpr (EXACT) {
        // first pass over the keys: the exact row max
#pragma unroll
        for (int i = 0; i < 4; ++i) dma_k(0, 0, i);
        for (int jt = 0; jt < nkt; ++jt) {
            const int buf = jt & 1, jn = min(jt + 1, nkt - 1);
            wait_vmcnt<0>();
            __syncthreads();
            scores(
                buf, [&](int g) __attribute__((always_inline)) {
                    if (g < 4) dma_k(buf ^ 1, jn, g);
                },
                true);
            mask_tail(jt);
#pragma unroll
            for (int qf = 0; qf < 4; ++qf) mu[qf] = fmaxf(mu[qf], tile_max(qf));
        }
        wait_vmcnt<0>();
        __syncthreads();  // every wave is done with the LDS tiles before they are refilled
    }

    v4f oacc[16][4];
#pragma unroll
    for (int df = 0; df < 16; ++df)
#pragma unroll
        for (int qf = 0; qf < 4; ++qf) oacc[df][qf] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // ---- softmax of the scores in s against mu, 16 pieces per query fragment qf, each small enough
    // to issue in the shadow of one MFMA of the previous tile's PV product: p = 2^((s - mu) C) in
    // fp32 for the row sums, bf16 for the MFMA (B operand of O^T += V^T P^T: positions 8 g + 4 kf + r
    // <- key 16 kf + 4 g + r)
    float tt[8], sa[4], mc;
    auto softmax_piece = [&](int qf, int i, v4u (&pn)[4]) __attribute__((always_inline)) {
        if (i < 4) {
            if (i == 0) mc = mu[qf] * C;
            tt[2 * i] = __builtin_fmaf(s[i / 2][qf][(2 * i) % 4], C, -mc);
            tt[2 * i + 1] = __builtin_fmaf(s[i / 2][qf][(2 * i) % 4 + 1], C, -mc);
        } else if (i < 12) {
            tt[i - 4] = __builtin_amdgcn_exp2f(tt[i - 4]);
        } else if (i == 12) {
            sa[0] = tt[0] + tt[1];
            sa[1] = tt[2] + tt[3];
            pn[qf][0] = pack_bf16x2(tt[0], tt[1]);
            pn[qf][1] = pack_bf16x2(tt[2], tt[3]);
        } else if (i == 13) {
            sa[2] = tt[4] + tt[5];
            sa[3] = tt[6] + tt[7];
            pn[qf][2] = pack_bf16x2(tt[4], tt[5]);
            pn[qf][3] = pack_bf16x2(tt[6], tt[7]);
        } else if (i == 14) {
            sa[0] = (sa[0] + sa[1]) + (sa[2] + sa[3]);
        } else {
            lp[qf] += sa[0];
        }
    };
    // ---- O^T += V^T P^T for the tile in V^T buffer vbuf (lane holds dims 16 df + 4 (lane >> 4) + r
    // of query 16 qf + (lane & 15)), each MFMA followed by one softmax piece of the current scores
    auto pv = [&](int vbuf, const v4u (&pp)[4], bool with_softmax, v4u (&pn)[4]) __attribute__((always_inline)) {
        asm volatile("s_nop 1");  // VALU-written P -> MFMA source
        v4u va[16];
#pragma unroll
        for (int df = 0; df < AT_LA; ++df) va[df] = vfrag(vbuf, df);
#pragma unroll
        for (int df = 0; df < 16; ++df) {
            if (df + AT_LA < 16) va[df + AT_LA] = vfrag(vbuf, df + AT_LA);
#pragma unroll
            for (int qf = 0; qf < 4; ++qf) {
                mfma_o(oacc[df][qf], va[df], pp[qf]);
                if (with_softmax) softmax_piece(df / 4, 4 * (df % 4) + qf, pn);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // V lags K by one tile: iteration jt computes the scores of tile jt and the PV product of tile
    // jt - 1, whose V^T arrived in the other V^T buffer one iteration earlier.  The LDS-DMAs of an
    // iteration (K of tile jt + 1, V^T of tile jt) run between its score MFMAs; tile indices past
    // the last are clamped rather than branched on.  The last PV product runs in one more
    // iteration (jt = nkt) whose scores are all masked to -inf, so that it adds nothing to the row
    // sums: a PV product outside the loop would have the compiler move the 256 accumulators to
    // other registers, right before MFMAs that read them.
    v4u pprev[4], pnew[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_k(0, 0, i);
    {
        wait_vmcnt<0>();
        __syncthreads();
        const int jn = min(1, nkt - 1);
        scores(
            0,
            [&](int g) __attribute__((always_inline)) {
                if (g < 4)
                    dma_k(1, jn, g);
                else if (g < 8)
                    dma_v(0, 0, g - 4);
            },
            true);
        mask_tail(0);
        if constexpr (!EXACT) {
            // the reference: the first tile's max
#pragma unroll
            for (int qf = 0; qf < 4; ++qf) mu[qf] = tile_max(qf);
        }
#pragma unroll
        for (int qf = 0; qf < 4; ++qf)
#pragma unroll
            for (int i = 0; i < 16; ++i) softmax_piece(qf, i, pprev);
    }
    // nkt >= 1.  The loop leaves only through the drain, so the register copies the compiler places
    // on its exit edge read finished accumulators.
    for (int jt = 1;; ++jt) {
        const int buf = jt & 1, jn = min(jt + 1, nkt - 1), jv = min(jt, nkt - 1);
        wait_vmcnt<0>();
        __syncthreads();
        scores(
            buf,
            [&](int g) __attribute__((always_inline)) {
                if (g < 4)
                    dma_k(buf ^ 1, jn, g);
                else if (g < 8)
                    dma_v(buf, jv, g - 4);
            },
            false);
        mask_tail(jt);
        pv(buf ^ 1, pprev, true, pnew);
#pragma unroll
        for (int qf = 0; qf < 4; ++qf) pprev[qf] = pnew[qf];
        if (jt == nkt) {
            mfma_drain();
            break;
        }
    }
    wait_vmcnt<0>();  // the last iteration's LDS-DMAs land before the workgroup ends
    if constexpr (!EXACT) {
        // a probability past 2^64 (a score more than 64 log2 units above the reference) leaves a
        // lane's partial row sum past 2^64: flag the workgroup for the exact-max rerun
        bool bad = false;
#pragma unroll
        for (int qf = 0; qf < 4; ++qf) bad |= !(lp[qf] <= 0x1p64f);
        if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) p.redo[t] = 1;
    }
    mfma_drain();
#pragma unroll
    for (int df = 0; df < 16; ++df)
#pragma unroll
        for (int qf = 0; qf < 4; ++qf) keep_after_a(oacc[df][qf]);

    // ---- normalize by the full row sums and store 4 consecutive dims per lane
#pragma unroll
    for (int qf = 0; qf < 4; ++qf) {
        float l = lp[qf];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const float inv = 1.0f / l;
        const int q = q0 + 16 * qf + (lane & 15);
        if (q >= p.S) continue;
        uint16_t* dst = p.O + (int64_t)q * p.ldo + h * AT_D + 4 * (lane >> 4);
#pragma unroll
        for (int df = 0; df < 16; ++df) {
            const v4f v = oacc[df][qf];
            *reinterpret_cast<uint2*>(dst + 16 * df) =
                make_uint2(pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv));
        }
    }
}

hipError_t launch_attention(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int S, int H, int64_t ld,
                            uint16_t* O, int64_t ldo, uint16_t* Vt, int* redo, hipStream_t st) {
    const int Spad = (S + AT_BK - 1) / AT_BK * AT_BK;
    const int tiles_q = (S + AT_BQ - 1) / AT_BQ;
    hipLaunchKernelGGL(attn_vt_kernel, dim3((Spad + 63) / 64, H), dim3(256), 0, st, V, ld, S, Spad, Vt, redo,
                       tiles_q * H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    AttnArgs a;
    a.Q = Q;
    a.K = K;
    a.Vt = Vt;
    a.O = O;
    a.ld = ld;
    a.ldo = ldo;
    a.S = S;
    a.Spad = Spad;
    a.H = H;
    a.tiles_q = tiles_q;
    a.redo = redo;
    hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3(tiles_q * H), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3(tiles_q * H), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace qdt
