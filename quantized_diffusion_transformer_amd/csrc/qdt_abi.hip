// The C ABI (include/qdt.h): argument validation, launch planning and kernel launches.
// Validation and planning are pure host code; nothing is enqueued unless every check passes.
#include <string.h>

#include <mutex>

#include "qdt_internal.h"

namespace qdt {

// Scratch of qdt_w8a8_linear_noalloc: the split-K partial sums live in this file-scope device
// array instead of a caller workspace.  Each device holds its own copy (allocated when the code
// object is loaded on it, kept until the process ends).  Host code never uses the array's name as
// a device address: the per-device address comes from hipGetSymbolAddress, taken once per device
// with that device current.
static __device__ __align__(256) uint8_t scratch[QDT_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call per device).
static hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Clock record of the W8A8 GEMM (qdt_clock_record): buffer, capacity and fill level in entries.
static std::mutex g_clk_mu;
static uint64_t* g_clk_buf = nullptr;
static int64_t g_clk_cap = 0, g_clk_used = 0;

uint64_t* clock_record_take(int grid) {
    std::lock_guard<std::mutex> lk(g_clk_mu);
    if (!g_clk_buf || g_clk_used + grid > g_clk_cap) return nullptr;
    uint64_t* p = g_clk_buf + 4 * g_clk_used;
    g_clk_used += grid;
    return p;
}

static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static inline bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

static inline qdt_status hip_status(hipError_t e) { return e == hipSuccess ? QDT_OK : QDT_EHIP; }

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Planner.  The GEMM keeps one 4-wave workgroup per compute unit, so the cost of a plan is
// (rounds of kNumCU workgroups) x (tile area) x (K steps per workgroup), plus the traffic of
// the split-K partial sums.  QDT_TILE_288 exists for the hidden width 4608 = 16 x 288: 256
// tiles at 4608 x 4608, exactly one per compute unit, where 256 x 256 tiles leave a second
// round that is only 68/256 full.
qdt_status make_plan(int64_t M, int64_t N, int64_t K, int epi, int esize, int tile_req, int split_req, Plan* p,
                     bool fp4) {
    const bool silu = epi == EPI_SILU, rms = epi == EPI_RMSNORM;
    Plan best{};
    double best_cost = -1.0;
    for (int tile = QDT_TILE_256; tile <= QDT_TILE_224x256; ++tile) {
        if (tile_req != QDT_TILE_AUTO && tile != tile_req) continue;
        if (tile == QDT_TILE_288 && (silu || rms)) continue;  // heads / gate-up halves need 256-wide tiles
        // 288 x 256 only on request: its weight and token waves issue unequal LDS-DMA counts and it
        // measured ~5% slower per FFN gate/up step than 256 x 256 despite fewer tile rounds
        if (tile == QDT_TILE_288x256 && tile_req == QDT_TILE_AUTO) continue;
        // 224 x 256 is an int8 tile (its 56 MFMA slots per K step hold too few for FP4's exponent
        // LDS-DMAs)
        if (tile == QDT_TILE_224x256 && (esize != 1 || fp4)) continue;
        const int bm = tile == QDT_TILE_256 ? 256 : tile == QDT_TILE_224x256 ? 224 : 288;  // token rows
        const int bn = tile == QDT_TILE_288 ? 288 : 256;                                   // weight rows
        const int64_t kstage = 128;  // bytes of K per main-loop stage (whole cache lines)
        const int64_t kt_total = cdiv(K * esize, kstage);
        const int64_t tiles_m = cdiv(M > 0 ? M : 1, bm);
        const int64_t tiles_n = silu ? cdiv(N / 2, bn / 2) : cdiv(N, bn);
        const int64_t tiles = tiles_m * tiles_n;
        int64_t split = 1;
        if (split_req > 0) {
            split = split_req;
        } else if (esize == 1 && tiles < kNumCU / 2 && kt_total * kstage >= 8192) {
            split = kNumCU / tiles;
            if (split > kt_total * kstage / 4096) split = kt_total * kstage / 4096;
            if (split > 16) split = 16;
            if (split < 1) split = 1;
        }
        if (split > kt_total) split = kt_total;
        const int64_t kps = cdiv(kt_total, split);
        split = cdiv(kt_total, kps);  // no empty slices
        const int64_t grid = tiles * split;
        const int64_t rounds = cdiv(grid, kNumCU);
        double cost = (double)rounds * bm * bn * kps * kstage / 8192.0;  // ~cycles of MFMA per CU
        // a 224-row tile moves 480 operand rows per stage for 7/8 of the MFMAs of a 256-row one
        if (tile == QDT_TILE_224x256) cost *= (480.0 / 512.0) / (224.0 / 256.0);
        if (split > 1) cost += (double)split * M * N * 4 * 2 / (8e12 / 2.4e9 / kNumCU) / kNumCU;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best.tile = tile;
            best.bm = bm;
            best.bn = bn;
            best.tiles_m = (int)tiles_m;
            best.tiles_n = (int)tiles_n;
            best.split_k = (int)split;
            best.kt_total = (int)kt_total;
            best.kt_per_split = (int)kps;
            best.grid = (int)grid;
            best.group_m = (int)(tiles_m < 4 ? tiles_m : 4);
            best.ws_bytes = split > 1 ? split * M * N * 4 : 0;
        }
    }
    if (best_cost < 0) return QDT_EUNSUPPORTED;
    *p = best;
    return QDT_OK;
}

}  // namespace qdt

using namespace qdt;

extern "C" {

const char* qdt_status_string(qdt_status s) {
    switch (s) {
        case QDT_OK: return "QDT_OK";
        case QDT_EINVAL: return "QDT_EINVAL: null pointer or invalid parameter";
        case QDT_ESHAPE: return "QDT_ESHAPE: unsupported dimension";
        case QDT_EALIGN: return "QDT_EALIGN: pointer or row stride not 16-byte aligned";
        case QDT_EWORKSPACE: return "QDT_EWORKSPACE: workspace missing or too small";
        case QDT_EALIAS: return "QDT_EALIAS: output overlaps an input";
        case QDT_EHIP: return "QDT_EHIP: HIP runtime error at launch";
        case QDT_EUNSUPPORTED: return "QDT_EUNSUPPORTED: no kernel for this request";
    }
    return "unknown qdt_status";
}

const char* qdt_version(void) { return "qdt 0.2 gfx950"; }

qdt_status qdt_clock_record(uint64_t* buf, int64_t entries) {
    if (buf && (entries <= 0 || (reinterpret_cast<uintptr_t>(buf) & 7u) != 0)) return QDT_EINVAL;
    std::lock_guard<std::mutex> lk(g_clk_mu);
    g_clk_buf = buf;
    g_clk_cap = buf ? entries : 0;
    g_clk_used = 0;
    return QDT_OK;
}

qdt_status qdt_clock_record_used(int64_t* entries) {
    if (!entries) return QDT_EINVAL;
    std::lock_guard<std::mutex> lk(g_clk_mu);
    *entries = g_clk_used;
    return QDT_OK;
}

qdt_status qdt_channel_absmax(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, float* s, int accumulate,
                              void* stream) {
    if (!s || (M > 0 && !X)) return QDT_EINVAL;
    if (M < 0 || K <= 0 || K % 8 != 0 || ldx < K) return QDT_ESHAPE;
    if (!aligned16(X) || !aligned16(s) || ldx % 8 != 0) return QDT_EALIGN;
    if (overlap(s, K * 4, X, M * ldx * 2)) return QDT_EALIAS;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (!accumulate) {
        qdt_status r = hip_status(launch_fill_f32(s, 0.0f, K, st));
        if (r != QDT_OK) return r;
    }
    return hip_status(launch_colmax(X, M, K, ldx, s, st));
}

qdt_status qdt_smooth_prepare(const uint16_t* W, const float* s, int64_t N, int64_t K, float alpha, int8_t* Wq,
                              float* w_scale, float* inv_lambda, float* lambda, void* stream) {
    if (!W || !Wq || !w_scale || !inv_lambda || !lambda) return QDT_EINVAL;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return QDT_EINVAL;
    if (N <= 0 || K <= 0 || K % 64 != 0 || K > QDT_MAX_K) return QDT_ESHAPE;
    if (!aligned16(W) || !aligned16(s) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(inv_lambda) ||
        !aligned16(lambda))
        return QDT_EALIGN;
    const void* ins[2] = {W, s};
    const int64_t inb[2] = {N * K * 2, s ? K * 4 : 0};
    void* outs[4] = {Wq, w_scale, inv_lambda, lambda};
    const int64_t outb[4] = {N * K, N * 4, K * 4, K * 4};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 2; ++i)
            if (overlap(outs[o], outb[o], ins[i], inb[i])) return QDT_EALIAS;
        for (int o2 = o + 1; o2 < 4; ++o2)
            if (overlap(outs[o], outb[o], outs[o2], outb[o2])) return QDT_EALIAS;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    qdt_status r;
    if (s) {
        // lambda holds w_j = max_n |W_nj| until the lambda kernel overwrites it
        if ((r = hip_status(launch_fill_f32(lambda, 0.0f, K, st))) != QDT_OK) return r;
        if ((r = hip_status(launch_colmax(W, N, K, K, lambda, st))) != QDT_OK) return r;
        if ((r = hip_status(launch_lambda(s, lambda, inv_lambda, K, alpha, st))) != QDT_OK) return r;
        return hip_status(launch_quant_rows(W, K, lambda, N, K, Wq, w_scale, st));
    }
    if ((r = hip_status(launch_fill_f32(lambda, 1.0f, K, st))) != QDT_OK) return r;
    if ((r = hip_status(launch_fill_f32(inv_lambda, 1.0f, K, st))) != QDT_OK) return r;
    return hip_status(launch_quant_rows(W, K, nullptr, N, K, Wq, w_scale, st));
}

qdt_status qdt_quantize_per_token(const uint16_t* X, const float* inv_lambda, int64_t M, int64_t K, int64_t ldx,
                                  int8_t* Xq, float* x_scale, void* stream) {
    if (M < 0) return QDT_ESHAPE;
    if (M > 0 && (!X || !Xq || !x_scale)) return QDT_EINVAL;
    if (K <= 0 || K % 64 != 0 || K > QDT_MAX_K || ldx < K || M > INT32_MAX) return QDT_ESHAPE;
    if (!aligned16(X) || !aligned16(inv_lambda) || !aligned16(Xq) || !aligned16(x_scale) || ldx % 8 != 0)
        return QDT_EALIGN;
    if (M == 0) return QDT_OK;
    const int64_t xb = ((M - 1) * ldx + K) * 2;
    if (overlap(Xq, M * K, X, xb) || overlap(Xq, M * K, inv_lambda, inv_lambda ? K * 4 : 0) ||
        overlap(x_scale, M * 4, X, xb) || overlap(x_scale, M * 4, inv_lambda, inv_lambda ? K * 4 : 0) ||
        overlap(x_scale, M * 4, Xq, M * K))
        return QDT_EALIAS;
    return hip_status(launch_quant_rows(X, ldx, inv_lambda, M, K, Xq, x_scale, reinterpret_cast<hipStream_t>(stream)));
}

qdt_status qdt_adaln_quantize(const uint16_t* X, int64_t ldx, const uint16_t* shift, const uint16_t* scale, float eps,
                              const float* inv_lambda, int64_t M, int64_t K, int8_t* Xq, float* x_scale, uint16_t* H,
                              void* stream) {
    if (M < 0) return QDT_ESHAPE;
    if (!(eps > 0.0f) || !(eps < INFINITY)) return QDT_EINVAL;
    // Xq and x_scale together, or neither (then only H is written, and H is required)
    if (M > 0 && (!X || (!Xq != !x_scale) || (!Xq && !H))) return QDT_EINVAL;
    if (K <= 0 || K % 64 != 0 || K > QDT_MAX_ADALN_K || ldx < K || M > INT32_MAX) return QDT_ESHAPE;
    if (!aligned16(X) || !aligned16(shift) || !aligned16(scale) || !aligned16(inv_lambda) || !aligned16(Xq) ||
        !aligned16(x_scale) || !aligned16(H) || ldx % 8 != 0)
        return QDT_EALIGN;
    if (M == 0) return QDT_OK;
    const int64_t xb = ((M - 1) * ldx + K) * 2;
    struct Span { const void* p; int64_t n; };
    const Span in[4] = {{X, xb}, {shift, shift ? K * 2 : 0}, {scale, scale ? K * 2 : 0},
                        {inv_lambda, inv_lambda ? K * 4 : 0}};
    const Span out[3] = {{Xq, M * K}, {x_scale, M * 4}, {H, H ? M * K * 2 : 0}};
    for (const Span& o : out) {
        for (const Span& i : in)
            if (overlap(o.p, o.n, i.p, i.n)) return QDT_EALIAS;
        for (const Span& o2 : out)
            if (&o2 != &o && overlap(o.p, o.n, o2.p, o2.n)) return QDT_EALIAS;
    }
    return hip_status(launch_adaln_quant(X, ldx, shift, scale, eps, inv_lambda, M, K, Xq, x_scale, H,
                                         reinterpret_cast<hipStream_t>(stream)));
}

qdt_status qdt_mxfp4_quantize(const uint16_t* X, const float* colmul, int64_t M, int64_t K, int64_t ldx, uint8_t* Q,
                              uint8_t* S, void* stream) {
    if (M < 0) return QDT_ESHAPE;
    if (M > 0 && (!X || !Q || !S)) return QDT_EINVAL;
    if (K <= 0 || K % 256 != 0 || K > QDT_MAX_K || ldx < K || M > INT32_MAX) return QDT_ESHAPE;
    if (!aligned16(X) || !aligned16(colmul) || !aligned16(Q) || ldx % 8 != 0) return QDT_EALIGN;
    if (M == 0) return QDT_OK;
    const int64_t xb = ((M - 1) * ldx + K) * 2, qb = M * K / 2, sb = M * K / 32;
    const int64_t cb = colmul ? K * 4 : 0;
    if (overlap(Q, qb, X, xb) || overlap(Q, qb, colmul, cb) || overlap(S, sb, X, xb) || overlap(S, sb, colmul, cb) ||
        overlap(S, sb, Q, qb))
        return QDT_EALIAS;
    return hip_status(launch_mx_quant(X, ldx, colmul, M, K, Q, S, reinterpret_cast<hipStream_t>(stream)));
}

static int epi_kind(qdt_epilogue e) {
    switch (e) {
        case QDT_EPI_BIAS: return EPI_BIAS;
        case QDT_EPI_SILU_GATE: return EPI_SILU;
        case QDT_EPI_HEAD_RMSNORM: return EPI_RMSNORM;
        case QDT_EPI_ACC_I32: return EPI_ACC;
        default: break;  // QDT_EPI_ACC_F32 belongs to the FP4 linear only
    }
    return -1;
}

static qdt_status check_shape(int64_t M, int64_t N, int64_t K, qdt_epilogue epi) {
    if (epi_kind(epi) < 0) return QDT_EINVAL;
    if (M < 0 || M > INT32_MAX / 2 || N <= 0 || N > INT32_MAX / 2 || N % 16 != 0) return QDT_ESHAPE;
    if (K <= 0 || K % 128 != 0 || K > QDT_MAX_K) return QDT_ESHAPE;
    if (epi == QDT_EPI_SILU_GATE && N % 32 != 0) return QDT_ESHAPE;
    if (epi == QDT_EPI_HEAD_RMSNORM && N % 256 != 0) return QDT_ESHAPE;
    return QDT_OK;
}

static void export_plan(const Plan& p, qdt_linear_plan* out) {
    out->tile = p.tile;
    out->split_k = p.split_k;
    out->tile_m = p.bm;
    out->tile_n = p.bn;
    out->tiles_m = p.tiles_m;
    out->tiles_n = p.tiles_n;
    out->k_tiles = p.kt_total;
    out->grid = p.grid;
    out->workspace_bytes = p.ws_bytes;
}

qdt_status qdt_w8a8_linear_plan(int64_t M, int64_t N, int64_t K, qdt_epilogue epi, qdt_linear_plan* plan) {
    if (!plan) return QDT_EINVAL;
    qdt_status r = check_shape(M, N, K, epi);
    if (r != QDT_OK) return r;
    Plan p;
    if ((r = make_plan(M, N, K, epi_kind(epi), 1, QDT_TILE_AUTO, 0, &p)) != QDT_OK) return r;
    export_plan(p, plan);
    return QDT_OK;
}

qdt_status qdt_w8a8_linear_plan_for(int64_t M, int64_t N, int64_t K, qdt_epilogue epi, int32_t tile, int32_t split_k,
                                    qdt_linear_plan* plan) {
    if (!plan) return QDT_EINVAL;
    qdt_status r = check_shape(M, N, K, epi);
    if (r != QDT_OK) return r;
    if (tile != QDT_TILE_AUTO && (tile < QDT_TILE_256 || tile > QDT_TILE_224x256)) return QDT_EINVAL;
    if (split_k < 0) return QDT_EINVAL;
    Plan p;
    if ((r = make_plan(M, N, K, epi_kind(epi), 1, tile, split_k, &p)) != QDT_OK) return r;
    export_plan(p, plan);
    return QDT_OK;
}

qdt_status qdt_w8a8_linear_workspace_size(int64_t M, int64_t N, int64_t K, qdt_epilogue epi, size_t* bytes) {
    if (!bytes) return QDT_EINVAL;
    qdt_linear_plan p;
    qdt_status r = qdt_w8a8_linear_plan(M, N, K, epi, &p);
    if (r != QDT_OK) return r;
    *bytes = (size_t)p.workspace_bytes;
    return QDT_OK;
}

static qdt_status linear_impl(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                              const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi,
                              const void* epi_params, void* Y, int64_t ldy, void* workspace, size_t workspace_bytes,
                              int tile_req, int split_req, qdt_linear_plan* plan_out, void* stream,
                              bool static_scratch = false) {
    qdt_status r = check_shape(M, N, K, epi);
    if (r != QDT_OK) return r;
    if (tile_req != QDT_TILE_AUTO && (tile_req < QDT_TILE_256 || tile_req > QDT_TILE_224x256)) return QDT_EINVAL;
    if (split_req < 0) return QDT_EINVAL;
    const int kind = epi_kind(epi);
    const qdt_rmsnorm_params* rp = reinterpret_cast<const qdt_rmsnorm_params*>(epi_params);
    if (epi == QDT_EPI_HEAD_RMSNORM) {
        if (!rp || !rp->gamma) return QDT_EINVAL;
        if (rp->head_dim != 256) return QDT_ESHAPE;
        if (!(rp->eps >= 0.0f) || rp->eps > 3.0e38f) return QDT_EINVAL;
        if (!aligned16(rp->gamma)) return QDT_EALIGN;
    }
    Plan p;
    if ((r = make_plan(M, N, K, kind, 1, tile_req, split_req, &p)) != QDT_OK) return r;
    if (plan_out) export_plan(p, plan_out);
    if (static_scratch && p.ws_bytes > QDT_NOALLOC_SCRATCH_BYTES) return QDT_EWORKSPACE;
    const int64_t nout = epi == QDT_EPI_SILU_GATE ? N / 2 : N;
    const int64_t ysz = epi == QDT_EPI_ACC_I32 ? 4 : 2;
    if (ldy < nout) return QDT_ESHAPE;
    if (M == 0) return QDT_OK;
    if (!Xq || !x_scale || !Wq || !w_scale || !Y) return QDT_EINVAL;
    if (!aligned16(Xq) || !aligned16(x_scale) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(bias) ||
        !aligned16(Y) || (ldy * ysz) % 16 != 0)
        return QDT_EALIGN;
    const int64_t ybytes = ((M - 1) * ldy + nout) * ysz;
    const void* ins[6] = {Xq, x_scale, Wq, w_scale, bias, rp && epi == QDT_EPI_HEAD_RMSNORM ? rp->gamma : nullptr};
    const int64_t inb[6] = {M * K, M * 4, N * K, N * 4, bias ? N * 2 : 0, 512};
    for (int i = 0; i < 6; ++i)
        if (overlap(Y, ybytes, ins[i], inb[i])) return QDT_EALIAS;
    if (static_scratch && p.ws_bytes > 0) {
        if ((r = hip_status(scratch_address(&workspace))) != QDT_OK) return r;
        workspace_bytes = QDT_NOALLOC_SCRATCH_BYTES;
    }
    if (p.ws_bytes > 0) {
        if (!workspace || (int64_t)workspace_bytes < p.ws_bytes) return QDT_EWORKSPACE;
        if (!aligned16(workspace)) return QDT_EALIGN;
        if (overlap(Y, ybytes, workspace, p.ws_bytes)) return QDT_EALIAS;
        for (int i = 0; i < 6; ++i)
            if (overlap(workspace, p.ws_bytes, ins[i], inb[i])) return QDT_EALIAS;
    }
    GemmArgs a;
    a.X = Xq;
    a.W = Wq;
    a.sx = x_scale;
    a.sw = w_scale;
    a.bias = bias;
    a.gamma = rp && epi == QDT_EPI_HEAD_RMSNORM ? rp->gamma : nullptr;
    a.eps = rp && epi == QDT_EPI_HEAD_RMSNORM ? rp->eps : 0.0f;
    a.Y = Y;
    a.ldy = ldy;
    a.ws = reinterpret_cast<int32_t*>(workspace);
    a.clk = clock_record_take(p.grid);
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.epi = kind;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if ((r = hip_status(launch_gemm_i8(a, p, st))) != QDT_OK) return r;
    if (p.split_k > 1) return hip_status(launch_splitk_epilogue(a, p.split_k, kind, st));
    return QDT_OK;
}

qdt_status qdt_w8a8_linear(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                           const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi,
                           const void* epi_params, void* Y, int64_t ldy, void* workspace, size_t workspace_bytes,
                           void* stream) {
    return linear_impl(Xq, x_scale, Wq, w_scale, bias, M, N, K, epi, epi_params, Y, ldy, workspace, workspace_bytes,
                       QDT_TILE_AUTO, 0, nullptr, stream);
}

qdt_status qdt_w8a8_linear_noalloc(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                                   const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi,
                                   const void* epi_params, void* Y, int64_t ldy, void* stream) {
    return linear_impl(Xq, x_scale, Wq, w_scale, bias, M, N, K, epi, epi_params, Y, ldy, nullptr, 0, QDT_TILE_AUTO,
                       0, nullptr, stream, true);
}

qdt_status qdt_w8a8_linear_planned(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                                   const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi,
                                   const void* epi_params, void* Y, int64_t ldy, void* workspace,
                                   size_t workspace_bytes, qdt_linear_plan* plan, void* stream) {
    if (!plan) return QDT_EINVAL;
    return linear_impl(Xq, x_scale, Wq, w_scale, bias, M, N, K, epi, epi_params, Y, ldy, workspace, workspace_bytes,
                       plan->tile, plan->split_k, plan, stream);
}

qdt_status qdt_bf16_linear(const uint16_t* X, const uint16_t* W, const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                           uint16_t* Y, int64_t ldy, void* stream) {
    if (M < 0 || M > INT32_MAX / 2 || N <= 0 || N > INT32_MAX / 2 || N % 16 != 0) return QDT_ESHAPE;
    if (K <= 0 || K % 64 != 0 || K > QDT_MAX_K || ldy < N) return QDT_ESHAPE;
    if (M == 0) return QDT_OK;
    if (!X || !W || !Y) return QDT_EINVAL;
    if (!aligned16(X) || !aligned16(W) || !aligned16(bias) || !aligned16(Y) || ldy % 8 != 0) return QDT_EALIGN;
    const int64_t ybytes = ((M - 1) * ldy + N) * 2;
    if (overlap(Y, ybytes, X, M * K * 2) || overlap(Y, ybytes, W, N * K * 2) || overlap(Y, ybytes, bias, bias ? N * 2 : 0))
        return QDT_EALIAS;
    Plan p;
    qdt_status r = make_plan(M, N, K, EPI_F32BIAS, 2, QDT_TILE_AUTO, 1, &p);
    if (r != QDT_OK) return r;
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.X = X;
    a.W = W;
    a.bias = bias;
    a.Y = Y;
    a.ldy = ldy;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.epi = EPI_F32BIAS;
    a.clk = clock_record_take(p.grid);
    return hip_status(launch_gemm_bf16(a, p, reinterpret_cast<hipStream_t>(stream)));
}

// The planner's view of an FP4 problem: K/2 code bytes per row, the int8 planner's tiles other
// than 224 x 256 and its K split rule (or the requested tile and split).
static qdt_status mx_plan(int64_t M, int64_t N, int64_t K, qdt_epilogue epi, int tile_req, int split_req, Plan* p) {
    if (epi != QDT_EPI_BIAS && epi != QDT_EPI_SILU_GATE && epi != QDT_EPI_HEAD_RMSNORM && epi != QDT_EPI_ACC_F32)
        return QDT_EINVAL;
    if (M < 0 || M > INT32_MAX / 2 || N <= 0 || N > INT32_MAX / 2 || N % 16 != 0) return QDT_ESHAPE;
    if (epi == QDT_EPI_SILU_GATE && N % 32 != 0) return QDT_ESHAPE;
    if (epi == QDT_EPI_HEAD_RMSNORM && N % 256 != 0) return QDT_ESHAPE;
    if (K <= 0 || K % 256 != 0 || K > QDT_MAX_K) return QDT_ESHAPE;
    if (tile_req != QDT_TILE_AUTO && (tile_req < QDT_TILE_256 || tile_req > QDT_TILE_288x256)) return QDT_EINVAL;
    if (split_req < 0) return QDT_EINVAL;
    const int pk = epi == QDT_EPI_SILU_GATE ? EPI_SILU : epi == QDT_EPI_HEAD_RMSNORM ? EPI_RMSNORM : EPI_BIAS;
    return make_plan(M, N, K / 2, pk, 1, tile_req, split_req, p, true);
}

qdt_status qdt_mxfp4_linear_plan(int64_t M, int64_t N, int64_t K, qdt_epilogue epi, qdt_linear_plan* plan) {
    if (!plan) return QDT_EINVAL;
    Plan p;
    qdt_status r = mx_plan(M, N, K, epi, QDT_TILE_AUTO, 0, &p);
    if (r == QDT_OK) export_plan(p, plan);
    return r;
}

qdt_status qdt_mxfp4_linear_plan_for(int64_t M, int64_t N, int64_t K, qdt_epilogue epi, int32_t tile, int32_t split_k,
                                     qdt_linear_plan* plan) {
    if (!plan) return QDT_EINVAL;
    Plan p;
    qdt_status r = mx_plan(M, N, K, epi, tile, split_k, &p);
    if (r == QDT_OK) export_plan(p, plan);
    return r;
}

static qdt_status mx_linear_impl(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                                 const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi,
                                 const void* epi_params, void* Y, int64_t ldy, void* workspace,
                                 size_t workspace_bytes, int tile_req, int split_req, qdt_linear_plan* plan_out,
                                 void* stream) {
    Plan p;
    qdt_status r = mx_plan(M, N, K, epi, tile_req, split_req, &p);
    if (r != QDT_OK) return r;
    if (plan_out) export_plan(p, plan_out);
    const qdt_rmsnorm_params* rp = reinterpret_cast<const qdt_rmsnorm_params*>(epi_params);
    if (epi == QDT_EPI_HEAD_RMSNORM) {
        if (!rp || !rp->gamma) return QDT_EINVAL;
        if (rp->head_dim != 256) return QDT_ESHAPE;
        if (!(rp->eps >= 0.0f) || rp->eps > 3.0e38f) return QDT_EINVAL;
        if (!aligned16(rp->gamma)) return QDT_EALIGN;
    }
    const int64_t nout = epi == QDT_EPI_SILU_GATE ? N / 2 : N;
    if (ldy < nout) return QDT_ESHAPE;
    if (M == 0) return QDT_OK;
    if (!Xq || !Xs || !Wq || !Ws || !Y) return QDT_EINVAL;
    if (!aligned16(Xq) || !aligned16(Wq) || !aligned16(bias) || !aligned16(Y) || ldy % 8 != 0 ||
        (reinterpret_cast<uintptr_t>(Xs) & 3u) != 0 || (reinterpret_cast<uintptr_t>(Ws) & 3u) != 0)
        return QDT_EALIGN;
    const int64_t es = epi == QDT_EPI_ACC_F32 ? 4 : 2;
    const int64_t ybytes = ((M - 1) * ldy + nout) * es;
    const void* ins[6] = {Xq, Xs, Wq, Ws, bias, epi == QDT_EPI_HEAD_RMSNORM ? rp->gamma : nullptr};
    const int64_t inb[6] = {M * K / 2, M * K / 32, N * K / 2, N * K / 32, bias ? N * 2 : 0, 512};
    for (int i = 0; i < 6; ++i)
        if (overlap(Y, ybytes, ins[i], inb[i])) return QDT_EALIAS;
    if (p.ws_bytes > 0) {
        if (!workspace || (int64_t)workspace_bytes < p.ws_bytes) return QDT_EWORKSPACE;
        if (!aligned16(workspace)) return QDT_EALIGN;
        if (overlap(Y, ybytes, workspace, p.ws_bytes)) return QDT_EALIAS;
        for (int i = 0; i < 6; ++i)
            if (overlap(workspace, p.ws_bytes, ins[i], inb[i])) return QDT_EALIAS;
    }
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.X = Xq;
    a.W = Wq;
    a.bias = bias;
    a.gamma = epi == QDT_EPI_HEAD_RMSNORM ? rp->gamma : nullptr;
    a.eps = epi == QDT_EPI_HEAD_RMSNORM ? rp->eps : 0.0f;
    a.Y = Y;
    a.ldy = ldy;
    a.ws = reinterpret_cast<int32_t*>(workspace);
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.epi = epi == QDT_EPI_ACC_F32         ? EPI_ACC
            : epi == QDT_EPI_SILU_GATE     ? EPI_F32SILU
            : epi == QDT_EPI_HEAD_RMSNORM  ? EPI_F32RMSNORM
                                           : EPI_F32BIAS;
    a.clk = clock_record_take(p.grid);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if ((r = hip_status(launch_gemm_mx(a, Xs, Ws, p, st))) != QDT_OK) return r;
    if (p.split_k > 1) return hip_status(launch_splitk_f32_epilogue(a, p.split_k, a.epi, st));
    return QDT_OK;
}

qdt_status qdt_mxfp4_linear(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                            const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi,
                            const void* epi_params, void* Y, int64_t ldy, void* workspace, size_t workspace_bytes,
                            void* stream) {
    return mx_linear_impl(Xq, Xs, Wq, Ws, bias, M, N, K, epi, epi_params, Y, ldy, workspace, workspace_bytes,
                          QDT_TILE_AUTO, 0, nullptr, stream);
}

qdt_status qdt_mxfp4_linear_planned(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                                    const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi,
                                    const void* epi_params, void* Y, int64_t ldy, void* workspace,
                                    size_t workspace_bytes, qdt_linear_plan* plan, void* stream) {
    if (!plan) return QDT_EINVAL;
    return mx_linear_impl(Xq, Xs, Wq, Ws, bias, M, N, K, epi, epi_params, Y, ldy, workspace, workspace_bytes,
                          plan->tile, plan->split_k, plan, stream);
}

// The weight-only linear's plan: 256 x 256 tiles and K slices of QDT_WO_KSLICE elements,
// whatever M is (the fixed reduction structure makes every output independent of M).
static qdt_status wo_plan(int64_t M, int64_t N, int64_t K, Plan* p) {
    if (M < 0 || M > INT32_MAX / 2 || N <= 0 || N > INT32_MAX / 2 || N % 16 != 0) return QDT_ESHAPE;
    if (K <= 0 || K % 512 != 0 || K > QDT_MAX_K) return QDT_ESHAPE;
    memset(p, 0, sizeof(*p));
    p->tile = QDT_TILE_256;
    p->bm = p->bn = 256;
    p->tiles_m = (int)cdiv(M, 256);
    p->tiles_n = (int)cdiv(N, 256);
    p->kt_total = (int)(K / 128);
    p->kt_per_split = QDT_WO_KSLICE / 128;
    p->split_k = (int)cdiv(p->kt_total, p->kt_per_split);
    p->group_m = 1;
    const int64_t grid = (int64_t)p->tiles_m * p->tiles_n * p->split_k;
    if (grid > INT32_MAX) return QDT_ESHAPE;
    p->grid = (int)grid;
    p->ws_bytes = p->split_k > 1 ? (int64_t)p->split_k * M * N * 4 : 0;
    return QDT_OK;
}

qdt_status qdt_wo_quantize(const uint16_t* W, int64_t N, int64_t K, int64_t ldw, int bits, uint8_t* Wq, uint16_t* Wd,
                           void* stream) {
    if (bits != 4 && bits != 8) return QDT_EINVAL;
    if (N < 0 || N > INT32_MAX) return QDT_ESHAPE;
    if (N > 0 && (!W || !Wq || !Wd)) return QDT_EINVAL;
    if (K <= 0 || K % 32 != 0 || K > QDT_MAX_K || ldw < K) return QDT_ESHAPE;
    if (!aligned16(W) || !aligned16(Wq) || (reinterpret_cast<uintptr_t>(Wd) & 1u) != 0 || ldw % 8 != 0)
        return QDT_EALIGN;
    if (N == 0) return QDT_OK;
    const int64_t wb = ((N - 1) * ldw + K) * 2, qb = N * K * bits / 8, db = N * (K / 32) * 2;
    if (overlap(Wq, qb, W, wb) || overlap(Wd, db, W, wb) || overlap(Wd, db, Wq, qb)) return QDT_EALIAS;
    return hip_status(launch_wo_quant(W, ldw, N, K, bits, Wq, Wd, reinterpret_cast<hipStream_t>(stream)));
}

qdt_status qdt_wo_linear_plan(int64_t M, int64_t N, int64_t K, qdt_linear_plan* plan) {
    if (!plan) return QDT_EINVAL;
    Plan p;
    qdt_status r = wo_plan(M, N, K, &p);
    if (r == QDT_OK) export_plan(p, plan);
    return r;
}

qdt_status qdt_wo_linear(const uint16_t* X, int64_t ldx, const uint8_t* Wq, const uint16_t* Wd, int bits,
                         const uint16_t* bias, int64_t M, int64_t N, int64_t K, qdt_epilogue epi, void* Y,
                         int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
    if (bits != 4 && bits != 8) return QDT_EINVAL;
    if (epi != QDT_EPI_BIAS && epi != QDT_EPI_ACC_F32) return QDT_EINVAL;
    Plan p;
    qdt_status r = wo_plan(M, N, K, &p);
    if (r != QDT_OK) return r;
    if (ldx < K || ldy < N) return QDT_ESHAPE;
    if (M == 0) return QDT_OK;
    if (!X || !Wq || !Wd || !Y) return QDT_EINVAL;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(bias) || !aligned16(Y) || ldx % 8 != 0 || ldy % 8 != 0 ||
        (reinterpret_cast<uintptr_t>(Wd) & 1u) != 0)
        return QDT_EALIGN;
    const int64_t es = epi == QDT_EPI_ACC_F32 ? 4 : 2;
    const int64_t ybytes = ((M - 1) * ldy + N) * es;
    const void* ins[4] = {X, Wq, Wd, bias};
    const int64_t inb[4] = {((M - 1) * ldx + K) * 2, N * K * bits / 8, N * (K / 32) * 2, bias ? N * 2 : 0};
    for (int i = 0; i < 4; ++i)
        if (overlap(Y, ybytes, ins[i], inb[i])) return QDT_EALIAS;
    if (p.ws_bytes > 0) {
        if (!workspace || (int64_t)workspace_bytes < p.ws_bytes) return QDT_EWORKSPACE;
        if (!aligned16(workspace)) return QDT_EALIGN;
        if (overlap(Y, ybytes, workspace, p.ws_bytes)) return QDT_EALIAS;
        for (int i = 0; i < 4; ++i)
            if (overlap(workspace, p.ws_bytes, ins[i], inb[i])) return QDT_EALIAS;
    }
    const int e = epi == QDT_EPI_ACC_F32 ? EPI_ACC : EPI_F32BIAS;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if ((r = hip_status(launch_wo_gemm(X, ldx, Wq, Wd, bits, bias, (int)M, (int)N, (int)K, e, Y, ldy,
                                       reinterpret_cast<float*>(workspace), p, st))) != QDT_OK)
        return r;
    if (p.split_k == 1) return QDT_OK;
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.bias = bias;
    a.Y = Y;
    a.ldy = ldy;
    a.ws = reinterpret_cast<int32_t*>(workspace);
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.epi = e;
    return hip_status(launch_splitk_f32_epilogue(a, p.split_k, e, st));
}

// Workspace: V^T per head (keys padded to a multiple of 32; only past kAttnVtrMaxS tokens, shorter
// sequences read V transposed in LDS), then 4 ints per workgroup (the waves' rerun flags), then the
// fp32 outputs of the key-range pieces (none unless the plan splits).
static int64_t attn_vt_bytes(int64_t S, int64_t H) {
    return attention_plan((int)S, (int)H).vtr ? 0 : H * QDT_ATTN_HEAD_DIM * ((S + 31) / 32 * 32) * 2;
}
static int64_t attn_redo_bytes(int64_t S, int64_t H) { return (int64_t)attention_plan((int)S, (int)H).workgroups * 16; }
static int64_t attn_ws_bytes(int64_t S, int64_t H) {
    return attn_vt_bytes(S, H) + attn_redo_bytes(S, H) + attention_plan((int)S, (int)H).part_floats * 4;
}

qdt_status qdt_attention_workspace_size(int64_t S, int64_t H, size_t* bytes) {
    if (!bytes) return QDT_EINVAL;
    if (S < 0 || S > QDT_ATTN_MAX_S || H <= 0 || H > 1024) return QDT_ESHAPE;
    *bytes = (size_t)attn_ws_bytes(S, H);
    return QDT_OK;
}

qdt_status qdt_attention(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t S, int64_t H, int64_t ld,
                         uint16_t* O, int64_t ldo, void* workspace, size_t workspace_bytes, void* stream) {
    if (S < 0 || S > QDT_ATTN_MAX_S || H <= 0 || H > 1024) return QDT_ESHAPE;
    if (ld < H * QDT_ATTN_HEAD_DIM || ldo < H * QDT_ATTN_HEAD_DIM) return QDT_ESHAPE;
    if (S == 0) return QDT_OK;
    if (!Q || !K || !V || !O) return QDT_EINVAL;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || ld % 8 != 0 || ldo % 8 != 0)
        return QDT_EALIGN;
    const int64_t wsb = attn_ws_bytes(S, H);
    if (!workspace || (int64_t)workspace_bytes < wsb) return QDT_EWORKSPACE;
    if (!aligned16(workspace)) return QDT_EALIGN;
    const int64_t inb = ((S - 1) * ld + H * QDT_ATTN_HEAD_DIM) * 2, ob = ((S - 1) * ldo + H * QDT_ATTN_HEAD_DIM) * 2;
    const void* ins[3] = {Q, K, V};
    for (int i = 0; i < 3; ++i)
        if (overlap(O, ob, ins[i], inb) || overlap(workspace, wsb, ins[i], inb)) return QDT_EALIAS;
    if (overlap(O, ob, workspace, wsb)) return QDT_EALIAS;
    uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
    return hip_status(launch_attention(Q, K, V, (int)S, (int)H, ld, O, ldo, reinterpret_cast<uint16_t*>(ws),
                                       reinterpret_cast<int*>(ws + attn_vt_bytes(S, H)),
                                       reinterpret_cast<float*>(ws + attn_vt_bytes(S, H) + attn_redo_bytes(S, H)),
                                       reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
