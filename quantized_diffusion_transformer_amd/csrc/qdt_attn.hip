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
// one dim row of V^T: 64 keys in the permuted order, zeros past S.  (Only for S past
// kAttnVtrMaxS; shorter sequences read V transposed from LDS instead.)
__global__ __launch_bounds__(256) void attn_vt_kernel(const uint16_t* __restrict__ V, int64_t ld, int S, int Spad,
                                                      uint16_t* __restrict__ Vt) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][AT_D];
    const int kb = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
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
    const uint16_t* Vt;  // V^T from attn_vt_kernel (VTR false)
    const uint16_t* V;   // V itself (VTR true)
    uint16_t* O;
    int* redo;    // per wave (4 per workgroup): scores outgrew the reference; written on every call
    float* part;  // key-range pieces: unnormalized O [piece][256 queries][256], then (m C, l) [piece][256][2]
    int64_t ld, ldo;
    int S, Spad, H, tiles_q;
    int t_full;   // workgroups 0 .. t_full-1 take whole (query block, head) tiles over all keys
    int split;    // each later tile is split over `split` key ranges (1: no later tiles)
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
// V rows, read transposed (512 bytes, 32 chunks; key r of the tile): chunk c in slot c ^ 2 (r mod 8).
// A transposing fragment read touches 16 key rows, 8 per half-wave, at chunks 2 df and 2 df + 1:
// each half-wave covers the 64 banks once (SQ_LDS_BANK_CONFLICT reads 0).
__device__ __forceinline__ int at_vsw2(int r) { return 2 * (r & 7); }
typedef short at_v4s __attribute__((ext_vector_type(4)));
typedef uint32_t at_u2 __attribute__((ext_vector_type(2)));

// Which workgroups a launch holds: the whole tiles or the key-range pieces.  (One launch holding
// both measured no faster for the rerun pass, and in the first pass the piece stores pushed the
// register allocation of a kernel holding both into spills.)
enum AttnWork { kWhole = 0, kPieces = 1 };

// VTR: the PV product reads V's rows transposed from LDS (ds_read_b64_tr_b16) instead of a V^T
// written by a separate pass.  Per tile that is two LDS reads per fragment instead of one and a few
// more VALU instructions (the main loop measured ~3% slower), against the V^T pass (~5.2 ns per
// token and head block of 18: 24 us of a 0.36 ms call at 4608 tokens, 88 us of 4.1 ms at 16896).
template <bool EXACT, int WORK, bool VTR>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void
attn_fwd_kernel(AttnArgs p) {
    constexpr int KROW = AT_D * 2;           // LDS bytes per key row
    constexpr int KT = AT_BK * KROW;         // 16 KiB K tile
    constexpr int VROW = AT_BK * 2;          // LDS bytes per V^T dim row
    constexpr int VT = AT_D * VROW;          // 16 KiB V^T tile
    constexpr int STG = KT + VT;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STG];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bid = blockIdx.x;
    const int nkt = p.Spad / AT_BK;
    // Work item of the workgroup.  Whole tiles (t_full of them, a whole number of rounds on the
    // compute units) run over all keys, dealt so that each XCD holds a contiguous run (one head's
    // tiles share K and V in its L2).  The remaining tiles would fill a last round only partly, so
    // each is split into `split` key ranges, one workgroup each; a range's unnormalized output and
    // its (reference, row sum) go to `part`, and attn_combine_kernel merges them.
    int t, kt0 = 0, kt1 = nkt, piece = -1;
    const int widx = WORK == kPieces ? p.t_full + bid : bid;  // index of the rerun flag
    if (WORK == kWhole) {
        const int nb = p.t_full;
        const int xcd = bid % kNumXCD, per = nb / kNumXCD, rem = nb % kNumXCD;
        t = xcd * per + min(xcd, rem) + bid / kNumXCD;
    } else {
        piece = bid;
        const int part = piece % p.split;
        t = p.t_full + piece / p.split;
        kt0 = part * nkt / p.split;
        kt1 = (part + 1) * nkt / p.split;
    }
    const int kend = min(p.S, kt1 * AT_BK);  // keys at or past kend are masked
    const int h = t / p.tiles_q, qt = t % p.tiles_q;
    const int q0 = qt * AT_BQ + 64 * wave;  // the wave's first query
    if constexpr (EXACT) {
        const int4 f = *reinterpret_cast<const int4*>(p.redo + 4 * widx);
        if (__builtin_amdgcn_readfirstlane(f.x | f.y | f.z | f.w) == 0) return;
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
    const uint8_t* vbase = VTR ? reinterpret_cast<const uint8_t*>(p.V + h * AT_D)
                               : reinterpret_cast<const uint8_t*>(p.Vt + (int64_t)h * AT_D * p.Spad);
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
    const uint32_t voff = VTR ? 0u : (uint32_t)((64 * wave + (lane >> 2)) * p.Spad * 2) +
                                     (uint32_t)(((lane & 3) ^ at_vsw(lane >> 2)) * 16);
    // VTR: V instruction i of this wave moves key rows 2 (4 w + i) + (lane >> 5), as for K, under
    // the V swizzle, its offset computed per instruction (an array of them would not fit)
    int vdrow = 8 * wave + (lane >> 5);
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
        if constexpr (VTR) {
            const int key0 = jt * AT_BK;
            asm volatile("" : "+v"(vdrow));
            const int row = vdrow + 2 * i;
            // rows past S read the last key: their probabilities are 0
            const uint32_t off = (uint32_t)(min(row, p.S - 1 - key0) * p.ld * 2) +
                                 (uint32_t)(((lane & 31) ^ at_vsw2(row)) * 16);
            lds_dma16_s(ldsv + (uint32_t)(buf * STG + i * 1024), off, vbase + (int64_t)key0 * p.ld * 2);
        } else {
            lds_dma16_s(ldsv + (uint32_t)(buf * STG + i * 1024), voff,
                        vbase + (int64_t)jt * AT_BK * 2 + (int64_t)16 * i * p.Spad * 2);
        }
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
    // VTR: the same fragment from the V rows, with two transposing reads.  In each 16-lane group g,
    // lane j points at dims 16 df + 4 (j & 3) .. + 3 of the key at position 8 g + 4 h + (j >> 2),
    // and lane i receives dim 16 df + i of the 4 keys at positions 8 g + 4 h .. + 3 (measured lane
    // layout: lane i gets element i & 3 of the chunks of lanes 4 k + (i >> 2), k = 0..3).  Position
    // 8 g + k (k < 4) holds key 4 g + k = lane >> 2 of the pointing lane, position 8 g + 4 + k key
    // 16 + (lane >> 2): the same row modulo 8, 16 rows (8 KiB) further.  The row offset has bits 5-7
    // clear, so the slot xor acts on the address: vrx = row offset | 32 (key mod 8), and dims
    // 16 df .. lie at (vrx ^ 32 (df mod 8)) + 256 (df / 8).
    uint32_t vrx = ((uint32_t)(KT + (lane >> 2) * KROW) + ((lane & 2) >> 1) * 16 + 8 * (lane & 1)) |
                   (32u * ((lane >> 2) & 7));
    auto vfrag_tr = [&](int buf, int df, uint32_t xa) __attribute__((always_inline)) {
        auto tr = [&](int hk) __attribute__((always_inline)) {
            const uint8_t* a = smem + buf * STG + hk * 16 * KROW + 256 * (df >> 3) + xa;
            return __builtin_bit_cast(at_u2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                 (__attribute__((address_space(3))) at_v4s*)(const_cast<uint8_t*>(a))));
        };
        const at_u2 lo = tr(0), hi = tr(1);
        v4u r;
        r[0] = lo.x;
        r[1] = lo.y;
        r[2] = hi.x;
        r[3] = hi.y;
        return r;
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
    // keys past S, or past the workgroup's key range, get -inf
    auto mask_tail = [&](int jt) __attribute__((always_inline)) {
        if ((jt + 1) * AT_BK > kend) {
            mfma_drain();
#pragma unroll
            for (int kf = 0; kf < 2; ++kf)
#pragma unroll
                for (int qf = 0; qf < 4; ++qf) keep_after_v(s[kf][qf]);
#pragma unroll
            for (int kf = 0; kf < 2; ++kf)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool out = jt * AT_BK + 16 * kf + 4 * (lane >> 4) + r >= kend;
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
        for (int i = 0; i < 4; ++i) dma_k(0, kt0, i);
        for (int jt = kt0; jt < kt1; ++jt) {
            const int buf = (jt - kt0) & 1, jn = min(jt + 1, kt1 - 1);
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
        // VTR: the fragments go in the order 0, 8, 1, 9, .., so that a pair shares its address
        // (each fragment has its own accumulators, so any order gives the same sums; the softmax
        // pieces keep their slots).  The address base is pinned here: hoisted out of the loop, the
        // per-read addresses would take registers the kernel does not have.
        if constexpr (VTR) asm volatile("" : "+v"(vrx));
        auto fdf = [](int n) { return VTR ? (n >> 1) + 8 * (n & 1) : n; };
        v4u va[16];
        uint32_t xa[VTR ? 8 : 1];
        auto load = [&](int n) __attribute__((always_inline)) {
            if constexpr (VTR) {
                if ((n & 1) == 0) xa[n >> 1] = vrx ^ (32u * (n >> 1));
                va[n] = vfrag_tr(vbuf, fdf(n), xa[n >> 1]);
            } else {
                va[n] = vfrag(vbuf, n);
            }
        };
#pragma unroll
        for (int n = 0; n < AT_LA; ++n) load(n);
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            if (n + AT_LA < 16) load(n + AT_LA);
            const int df = fdf(n);
#pragma unroll
            for (int qf = 0; qf < 4; ++qf) {
                mfma_o(oacc[df][qf], va[n], pp[qf]);
                if (with_softmax) softmax_piece(n / 4, 4 * (n % 4) + qf, pn);
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
    for (int i = 0; i < 4; ++i) dma_k(0, kt0, i);
    {
        wait_vmcnt<0>();
        __syncthreads();
        const int jn = min(kt0 + 1, kt1 - 1);
        scores(
            0,
            [&](int g) __attribute__((always_inline)) {
                if (g < 4)
                    dma_k(1, jn, g);
                else if (g < 8)
                    dma_v(0, kt0, g - 4);
            },
            true);
        mask_tail(kt0);
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
    // kt1 > kt0.  The loop leaves only through the drain, so the register copies the compiler places
    // on its exit edge read finished accumulators.
    for (int lj = 1;; ++lj) {
        const int jt = kt0 + lj;
        const int buf = lj & 1, jn = min(jt + 1, kt1 - 1), jv = min(jt, kt1 - 1);
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
        if (jt == kt1) {
            mfma_drain();
            break;
        }
    }
    wait_vmcnt<0>();  // the last iteration's LDS-DMAs land before the workgroup ends
    if constexpr (!EXACT) {
        // a probability past 2^64 (a score more than 64 log2 units above the reference) leaves a
        // lane's partial row sum past 2^64: flag the wave for the exact-max rerun (each wave writes
        // its flag on every call, so no pass has to clear them)
        bool bad = false;
#pragma unroll
        for (int qf = 0; qf < 4; ++qf) bad |= !(lp[qf] <= 0x1p64f);
        const bool any = __builtin_amdgcn_ballot_w64(bad) != 0;
        if (lane == 0) p.redo[4 * widx + wave] = any ? 1 : 0;
    }
    mfma_drain();
#pragma unroll
    for (int df = 0; df < 16; ++df)
#pragma unroll
        for (int qf = 0; qf < 4; ++qf) keep_after_a(oacc[df][qf]);

    if (WORK == kPieces) {
        // a key-range piece: its unnormalized output, its reference m C and row sum per query
        float* po = p.part + (int64_t)piece * AT_BQ * AT_D;
        float* pml = p.part + (int64_t)(p.H * p.tiles_q - p.t_full) * p.split * AT_BQ * AT_D + (int64_t)piece * AT_BQ * 2;
#pragma unroll
        for (int qf = 0; qf < 4; ++qf) {
            float l = lp[qf];
            l += __shfl_xor(l, 16, 64);
            l += __shfl_xor(l, 32, 64);
            const int ql = 64 * wave + 16 * qf + (lane & 15);  // query within the tile
            float* dst = po + (int64_t)ql * AT_D + 4 * (lane >> 4);
            // one accumulator tuple at a time: reading all 16 first would need 64 more VGPRs
#pragma unroll
            for (int df = 0; df < 16; ++df) {
                *reinterpret_cast<v4f*>(dst + 16 * df) = oacc[df][qf];
                __builtin_amdgcn_sched_barrier(0);
            }
            if ((lane >> 4) == 0) {
                pml[2 * ql] = mu[qf] * C;
                pml[2 * ql + 1] = l;
            }
        }
    } else {
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
}

// ---------------------------------------------------------------------------- combine
// Merges the key-range pieces of a split tile: with the pieces' references c_i = m_i C (log2 units)
// and row sums l_i, M = max c_i, w_i = 2^(c_i - M), O = (sum_i w_i O_i) / (sum_i w_i l_i), summed
// in piece order.  One thread per 4 dims of a query, 4 queries per block.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs p) {
    const int64_t npieces = (int64_t)(p.H * p.tiles_q - p.t_full) * p.split;
    const int per_tile = AT_BQ / 4;
    const int tt = blockIdx.x / per_tile;
    const int ql = (blockIdx.x % per_tile) * 4 + (threadIdx.x >> 6);
    const int d = (threadIdx.x & 63) * 4;
    const int t = p.t_full + tt;
    const int h = t / p.tiles_q, q = (t % p.tiles_q) * AT_BQ + ql;
    if (q >= p.S) return;
    const float* ml = p.part + npieces * AT_BQ * AT_D;
    float m = -__builtin_inff();
    for (int i = 0; i < p.split; ++i) m = fmaxf(m, ml[((int64_t)(tt * p.split + i) * AT_BQ + ql) * 2]);
    float l = 0.0f;
    v4f o = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int i = 0; i < p.split; ++i) {
        const int64_t pc = (int64_t)tt * p.split + i;
        const float w = __builtin_amdgcn_exp2f(ml[(pc * AT_BQ + ql) * 2] - m);
        l += w * ml[(pc * AT_BQ + ql) * 2 + 1];
        const v4f v = *reinterpret_cast<const v4f*>(p.part + (pc * AT_BQ + ql) * AT_D + d);
        o += w * v;
    }
    const float inv = 1.0f / l;
    *reinterpret_cast<uint2*>(p.O + (int64_t)q * p.ldo + h * AT_D + d) =
        make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
}

// A last round of workgroups that would be less than half full (R tiles past a whole number of
// rounds, R <= kNumCU / 2) is replaced by R x floor(kNumCU / R) key-range pieces, which fill it.
AttnPlan attention_plan(int S, int H) {
    AttnPlan pl;
    const int tiles_q = (S + AT_BQ - 1) / AT_BQ;
    const int nkt = (S + AT_BK - 1) / AT_BK;
    pl.tiles = tiles_q * H;
    const int r = pl.tiles % kNumCU;
    int split = r > 0 && pl.tiles > kNumCU ? kNumCU / r : 1;
    if (split > nkt) split = nkt;  // every piece holds at least one key tile
    if (split < 2) split = 1;
    pl.split = split;
    pl.t_full = split > 1 ? pl.tiles - r : pl.tiles;
    pl.workgroups = pl.t_full + (pl.tiles - pl.t_full) * split;
    pl.part_floats = split > 1 ? (int64_t)(pl.tiles - pl.t_full) * split * AT_BQ * (AT_D + 2) : 0;
    pl.vtr = S <= kAttnVtrMaxS;
    return pl;
}

template <bool VTR>
static hipError_t launch_attention_as(const AttnPlan& pl, const AttnArgs& a, hipStream_t st) {
    hipError_t e;
    const int npieces = (pl.tiles - pl.t_full) * pl.split;
    hipLaunchKernelGGL((attn_fwd_kernel<false, kWhole, VTR>), dim3(pl.t_full), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (npieces > 0) {
        hipLaunchKernelGGL((attn_fwd_kernel<false, kPieces, VTR>), dim3(npieces), dim3(256), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((attn_fwd_kernel<true, kWhole, VTR>), dim3(pl.t_full), dim3(256), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((attn_fwd_kernel<true, kPieces, VTR>), dim3(npieces), dim3(256), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(attn_combine_kernel, dim3((pl.tiles - pl.t_full) * (AT_BQ / 4)), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((attn_fwd_kernel<true, kWhole, VTR>), dim3(pl.t_full), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_attention(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int S, int H, int64_t ld,
                            uint16_t* O, int64_t ldo, uint16_t* Vt, int* redo, float* part, hipStream_t st) {
    const int Spad = (S + AT_BK - 1) / AT_BK * AT_BK;
    const int tiles_q = (S + AT_BQ - 1) / AT_BQ;
    const AttnPlan pl = attention_plan(S, H);
    if (!pl.vtr) {
        hipLaunchKernelGGL(attn_vt_kernel, dim3((Spad + 63) / 64, H), dim3(256), 0, st, V, ld, S, Spad, Vt);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    AttnArgs a;
    a.Q = Q;
    a.K = K;
    a.Vt = Vt;
    a.V = V;
    a.O = O;
    a.ld = ld;
    a.ldo = ldo;
    a.S = S;
    a.Spad = Spad;
    a.H = H;
    a.tiles_q = tiles_q;
    a.redo = redo;
    a.part = part;
    a.t_full = pl.t_full;
    a.split = pl.split;
    return pl.vtr ? launch_attention_as<true>(pl, a, st) : launch_attention_as<false>(pl, a, st);
}

}  // namespace qdt
