"""Parity of the block-scaled FP4 (MXFP4) path against the oracle.

The quantizer's codes and block exponents are gated bit for bit.  The GEMM is gated bit for bit
on inputs whose partial sums are exact in fp32 (any summation order gives the exact sum), which
pins the fragment layout, the nibble order and the placement of every block exponent.  On
general inputs its bf16 output is gated by 1 bf16 ulp plus the fp32 summation bound
gamma_K * sum_k |x_k w_k| of the decoded values (carried through silu(g) u for the gated SiLU).
"""
import numpy as np
import pytest

import oracle
import qdt_workloads as W
from qdt_testutil import (bits_equal, mx_exponents_from_rows, mx_exponents_to_rows, sample_rows, to_dev, to_host,
                          ulp_bf16)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
qdt = pytest.importorskip("quantized_diffusion_transformer_amd")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def ex_host(S):
    """Library-layout exponents on the device -> the oracle's row-major [rows, K/32]."""
    return mx_exponents_to_rows(to_host(S))


def ex_dev(S):
    """Row-major [rows, K/32] exponents (oracle layout) -> library layout on the device."""
    return to_dev(mx_exponents_from_rows(S))


def check_quant(X, colmul=None, ldx=None):
    M, K = X.shape
    Xh = X
    if ldx is not None:
        Xh = np.full((M, ldx), 0x7FC0, np.uint16)  # NaN padding: must never be read
        Xh[:, :K] = X
    Xd = to_dev(Xh)[:, :K] if ldx is not None else to_dev(Xh)
    Q, S = qdt.mxfp4_quantize(Xd, None if colmul is None else to_dev(colmul))
    torch.cuda.synchronize()
    Qr, Sr = oracle.mxfp4_quantize(X, colmul)
    Qg, Sg = to_host(Q), ex_host(S)
    assert bits_equal(Sg, Sr), f"exponents: {np.sum(Sg != Sr)} differ"
    assert bits_equal(Qg, Qr), f"codes: {np.sum(Qg != Qr)} bytes differ"
    return Q, S


@pytest.mark.parametrize("M,K", [(1, 256), (37, 512), (300, 4608), (5, 53248)])
def test_mxfp4_quantize_parity(M, K):
    announce(f"mxfp4_quantize M={M} K={K}")
    X = W.activations(M, K, 4000 + K, "pct1")
    check_quant(X)
    inv = (np.random.default_rng(K).uniform(0.05, 3.0, K)).astype(np.float32)
    check_quant(X, inv)


def test_mxfp4_quantize_special_blocks_and_stride():
    announce("mxfp4_quantize special blocks, ldx > K")
    rng = np.random.default_rng(41)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    x[0, :32] = 0.0                                   # zero block
    x[1, 32:64] = 1e-39 * rng.standard_normal(32)     # subnormal block maximum
    x[2, 64:96] = 3e38 * np.sign(rng.standard_normal(32))  # exponent near the top
    x[3, :32] = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.75, -0.25, -0.1, -5.0] + [0.0] * 19
    x[4] = -1e-3 * np.abs(rng.standard_normal(512))   # negative values, some rounding to zero
    x[4, ::32] = -1.0
    check_quant(W.f32_to_bf16_bits(x), ldx=512 + 40)


def exact_operands(rows, K, seed):
    """Random codes with block exponents in {-2, -1, 0}: every product is a multiple of 2^-6
    below 36, so sums over K <= 1024 stay exact in fp32."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, (rows, K))
    codes[codes == 8] = 0  # canonical zero
    Q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    S = rng.integers(125, 128, (rows, K // 32)).astype(np.uint8)
    return Q, S


@pytest.mark.parametrize("M,N,K", [(16, 16, 256), (300, 272, 512), (513, 256, 1024)])
def test_mxfp4_gemm_exact_accumulators(M, N, K):
    announce(f"mxfp4_linear exact M={M} N={N} K={K}")
    Xq, Xs = exact_operands(M, K, 50 + M)
    Wq, Ws = exact_operands(N, K, 60 + N)
    _, acc = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, want_acc=True)
    Y = to_host(qdt.mxfp4_linear(to_dev(Xq), ex_dev(Xs), to_dev(Wq), ex_dev(Ws), None, "acc_f32"))
    assert np.array_equal(Y.astype(np.float64), acc), f"{np.sum(Y != acc)} accumulators differ"


def within_bound(Y, Xq, Xs, Wq, Ws, bias, rows):
    Y_ref, acc = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias, rows, want_acc=True)
    xd = oracle.mxfp4_dequantize(Xq[rows], Xs[rows])
    wd = oracle.mxfp4_dequantize(Wq, Ws)
    K = xd.shape[1]
    gam = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
    b = 0.0 if bias is None else W.bf16_bits_to_f32(bias).astype(np.float64)
    ref = acc + b
    bound = gam * (np.abs(xd) @ np.abs(wd).T) + 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    got = W.bf16_bits_to_f32(Y[rows]).astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"worst error / bound {np.max(err / bound):.3f}"
    return float(np.mean(Y[rows] == Y_ref))


@pytest.mark.parametrize("M,N,K", [(64, 128, 256), (300, 4608, 4608)])
def test_mxfp4_linear_bias_within_bound(M, N, K):
    announce(f"mxfp4_linear bias M={M} N={N} K={K}")
    d = W.make_linear(M, N, K, seed=4100 + M, x_kind="pct1", w_sigma=0.015, bias=True)
    Xq, Xs = check_quant(d["X"])
    Wq, Ws = check_quant(d["W"])
    Y = to_host(qdt.mxfp4_linear(Xq, Xs, Wq, Ws, to_dev(d["bias"]), "bias"))
    rows = np.arange(M) if M <= 64 else sample_rows(M, 24, 5)
    exact = within_bound(Y, to_host(Xq), ex_host(Xs), to_host(Wq), ex_host(Ws), d["bias"], rows)
    assert exact > 0.9, f"only {exact:.3f} of the outputs equal the correctly rounded result"


def test_mxfp4_attention_projection_4608():
    """The headline shape in block-scaled FP4, sampled rows, in the benchmark's launch."""
    announce("mxfp4 4608x4608x4608")
    d = W.make_workload("dit_attn_proj_4608x4608x4608")
    Xq, Xs = qdt.mxfp4_quantize(to_dev(d["X"]))
    Wq, Ws = qdt.mxfp4_quantize(to_dev(d["W"]))
    Y = to_host(qdt.mxfp4_linear(Xq, Xs, Wq, Ws, to_dev(d["bias"]), "bias"))
    rows = sample_rows(4608, 16, 6)
    Qr, Sr = oracle.mxfp4_quantize(d["X"][rows])
    assert bits_equal(to_host(Xq)[rows], Qr) and bits_equal(ex_host(Xs)[rows], Sr)
    Wqr, Wsr = oracle.mxfp4_quantize(d["W"])
    assert bits_equal(to_host(Wq), Wqr) and bits_equal(ex_host(Ws), Wsr)
    Xqh, Xsh = to_host(Xq), ex_host(Xs)
    within_bound(Y, Xqh, Xsh, Wqr, Wsr, d["bias"], rows)


@pytest.mark.parametrize("M,F,K", [(300, 272, 512), (64, 128, 1024)])
def test_mxfp4_silu_gate_exact_sums_within_one_ulp(M, F, K):
    """With sums exact in fp32, g and u equal the oracle's, so only the exponential and the
    reciprocal can differ: the output is gated at 1 bf16 ulp, like the W8A8 gate."""
    announce(f"mxfp4_linear silu_gate exact sums M={M} F={F} K={K}")
    Xq, Xs = exact_operands(M, K, 70 + M)
    Wq, Ws = exact_operands(2 * F, K, 80 + F)
    bias = W.f32_to_bf16_bits(np.random.default_rng(F).standard_normal(2 * F).astype(np.float32) * 4)
    Y_ref = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias, epi="silu_gate")
    Y = to_host(qdt.mxfp4_linear(to_dev(Xq), ex_dev(Xs), to_dev(Wq), ex_dev(Ws), to_dev(bias), "silu_gate"))
    assert Y.shape == (M, F)
    u = ulp_bf16(Y, Y_ref)
    assert u.max() <= 1, f"max ulp {u.max()}"


@pytest.mark.parametrize("M,F,K", [(300, 1024, 4608)])
def test_mxfp4_silu_gate_within_bound(M, F, K):
    """General inputs: the fp32 accumulation error of g and u carried through silu(g) u
    (|silu'| <= 1.1), plus the fast exponential's relative error and one bf16 ulp."""
    announce(f"mxfp4_linear silu_gate M={M} F={F} K={K}")
    d = W.make_linear(M, 2 * F, K, seed=4200 + M, x_kind="pct1", w_sigma=0.015, bias=True)
    Xq, Xs = check_quant(d["X"])
    Wq, Ws = check_quant(d["W"])
    Y = to_host(qdt.mxfp4_linear(Xq, Xs, Wq, Ws, to_dev(d["bias"]), "silu_gate"))
    rows = sample_rows(M, 24, 8)
    Xqh, Xsh, Wqh, Wsh = to_host(Xq), ex_host(Xs), to_host(Wq), ex_host(Ws)
    Y_ref, acc = oracle.mxfp4_gemm_rows(Xqh, Xsh, Wqh, Wsh, d["bias"], rows, want_acc=True, epi="silu_gate")
    xd = np.abs(oracle.mxfp4_dequantize(Xqh[rows], Xsh[rows]))
    wd = np.abs(oracle.mxfp4_dequantize(Wqh, Wsh))
    gam = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
    b = W.bf16_bits_to_f32(d["bias"]).astype(np.float64)
    ga, ua = acc[:, :F] + b[:F], acc[:, F:] + b[F:]
    dg = gam * (xd @ wd[:F].T) + np.abs(ga) * 2.0 ** -23
    du = gam * (xd @ wd[F:].T) + np.abs(ua) * 2.0 ** -23
    silu = ga / (1.0 + np.exp(-ga))
    ref = silu * ua
    bound = 1.1 * dg * (np.abs(ua) + du) + np.abs(silu) * du + 1e-5 * np.abs(ref) \
        + 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    got = W.bf16_bits_to_f32(Y[rows]).astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"worst error / bound {np.max(err / bound):.3f}"
    assert np.mean(Y[rows] == Y_ref) > 0.9


@pytest.mark.parametrize("M,N,K", [(300, 512, 512), (64, 256, 1024)])
def test_mxfp4_head_rmsnorm_exact_sums_within_one_ulp(M, N, K):
    """With sums exact in fp32 the per-head statistics differ only in summation order."""
    announce(f"mxfp4_linear head_rmsnorm exact sums M={M} N={N} K={K}")
    Xq, Xs = exact_operands(M, K, 90 + M)
    Wq, Ws = exact_operands(N, K, 100 + N)
    rng = np.random.default_rng(N)
    bias = W.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    gamma = W.f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(256)).astype(np.float32))
    Y_ref = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias, epi="head_rmsnorm", gamma=gamma, eps=1e-6)
    Y = to_host(qdt.mxfp4_linear(to_dev(Xq), ex_dev(Xs), to_dev(Wq), ex_dev(Ws), to_dev(bias), "head_rmsnorm",
                                 gamma=to_dev(gamma), eps=1e-6))
    u = ulp_bf16(Y, Y_ref)
    assert u.max() <= 1, f"max ulp {u.max()}"


def test_mxfp4_head_rmsnorm_within_bound():
    """General inputs: the fp32 accumulation error of y carried through the per-head normalization."""
    M, N, K = 300, 4608, 4608
    announce(f"mxfp4_linear head_rmsnorm M={M} N={N} K={K}")
    d = W.make_linear(M, N, K, seed=4300, x_kind="pct1", w_sigma=0.015, bias=True, epi="head_rmsnorm")
    Xq, Xs = check_quant(d["X"])
    Wq, Ws = check_quant(d["W"])
    Y = to_host(qdt.mxfp4_linear(Xq, Xs, Wq, Ws, to_dev(d["bias"]), "head_rmsnorm", gamma=to_dev(d["gamma"]),
                                 eps=d["eps"]))
    rows = sample_rows(M, 16, 10)
    Xqh, Xsh, Wqh, Wsh = to_host(Xq), ex_host(Xs), to_host(Wq), ex_host(Ws)
    Y_ref, acc = oracle.mxfp4_gemm_rows(Xqh, Xsh, Wqh, Wsh, d["bias"], rows, want_acc=True, epi="head_rmsnorm",
                                        gamma=d["gamma"], eps=d["eps"])
    xd = np.abs(oracle.mxfp4_dequantize(Xqh[rows], Xsh[rows]))
    wd = np.abs(oracle.mxfp4_dequantize(Wqh, Wsh))
    gam = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
    y = acc + W.bf16_bits_to_f32(d["bias"]).astype(np.float64)
    dy = gam * (xd @ wd.T) + np.abs(y) * 2.0 ** -23
    g = W.bf16_bits_to_f32(d["gamma"]).astype(np.float64)
    got = W.bf16_bits_to_f32(Y[rows]).astype(np.float64)
    for h in range(N // 256):
        sl = slice(h * 256, (h + 1) * 256)
        yh, dyh = y[:, sl], dy[:, sl]
        ms = (yh ** 2).mean(axis=1, keepdims=True) + d["eps"]
        r = 1.0 / np.sqrt(ms)
        ref = yh * r * g
        dr = r * (np.abs(yh) * dyh).mean(axis=1, keepdims=True) / ms + r * 2.0 ** -21  # first order, plus fp32 ops
        bound = 2.0 * np.abs(g) * (dyh * r + np.abs(yh) * dr) \
            + 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
        err = np.abs(got[:, sl] - ref)
        assert np.all(err <= bound), f"head {h}: worst error / bound {np.max(err / bound):.3f}"
    assert np.mean(Y[rows] == Y_ref) > 0.9


def small_operands(rows, K, seed):
    """Codes of magnitude <= 1 with block exponents in {-1, 0}: every product is a multiple of 2^-4
    at most 1, so sums over K <= 53248 (and any split of them) stay exact in fp32."""
    rng = np.random.default_rng(seed)
    codes = rng.choice(np.array([0, 1, 2, 9, 10]), (rows, K))
    Q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    S = rng.integers(126, 128, (rows, K // 32)).astype(np.uint8)
    return Q, S


@pytest.mark.parametrize("M,N,K", [(300, 512, 16384), (64, 256, 53248)])
def test_mxfp4_split_k_exact(M, N, K):
    """Deep K: the planner splits K, the slices write fp32 partials and a second kernel sums them.
    With exact sums every epilogue must match the oracle (bias bit for bit, SiLU / RMSNorm 1 ulp)."""
    plan = qdt.mxfp4_linear_plan(M, N, K)
    assert plan["split_k"] > 1
    announce(f"mxfp4_linear split-K {plan['split_k']} M={M} N={N} K={K}")
    Xq, Xs = small_operands(M, K, 110 + M)
    Wq, Ws = small_operands(N, K, 120 + N)
    rng = np.random.default_rng(K)
    bias = W.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    gamma = W.f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(256)).astype(np.float32))
    dX, dXs, dW, dWs, db = to_dev(Xq), ex_dev(Xs), to_dev(Wq), ex_dev(Ws), to_dev(bias)
    Y_ref, acc = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias, want_acc=True)
    Yacc = to_host(qdt.mxfp4_linear(dX, dXs, dW, dWs, None, "acc_f32"))
    assert np.array_equal(Yacc.astype(np.float64), acc), f"{np.sum(Yacc != acc)} accumulators differ"
    assert bits_equal(to_host(qdt.mxfp4_linear(dX, dXs, dW, dWs, db, "bias")), Y_ref)
    Ys = to_host(qdt.mxfp4_linear(dX, dXs, dW, dWs, db, "silu_gate"))
    assert ulp_bf16(Ys, oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias, epi="silu_gate")).max() <= 1
    Yr = to_host(qdt.mxfp4_linear(dX, dXs, dW, dWs, db, "head_rmsnorm", gamma=to_dev(gamma), eps=1e-6))
    Yr_ref = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias, epi="head_rmsnorm", gamma=gamma, eps=1e-6)
    assert ulp_bf16(Yr, Yr_ref).max() <= 1


def test_mxfp4_text_projection_shape():
    """The deep-K text projection (512 x 4608 x 53248) in FP4 with its K split, sampled rows."""
    d = W.make_workload("text_cond_proj_512x4608x53248")
    plan = qdt.mxfp4_linear_plan(512, 4608, 53248)
    announce(f"mxfp4 text projection, split-K {plan['split_k']}")
    Xq, Xs = check_quant(d["X"])
    Wq, Ws = qdt.mxfp4_quantize(to_dev(d["W"]))
    Y = to_host(qdt.mxfp4_linear(Xq, Xs, Wq, Ws, to_dev(d["bias"]), "bias"))
    within_bound(Y, to_host(Xq), ex_host(Xs), to_host(Wq), ex_host(Ws), d["bias"], sample_rows(512, 4, 11))


MX_TILES = [(qdt.QDT_TILE_256, "256x256"), (qdt.QDT_TILE_288, "288x288"), (qdt.QDT_TILE_288x256, "288x256")]


@pytest.mark.parametrize("tile,tname", MX_TILES, ids=[t[1] for t in MX_TILES])
@pytest.mark.parametrize("M,N,K", [(16, 16, 256), (170, 288, 256), (300, 272, 512), (600, 592, 1024)])
def test_mxfp4_tiles_exact_accumulators(tile, tname, M, N, K):
    """Every FP4 tile on exact-sum inputs, M and N ragged against it (170 rows end inside the
    second exponent block copy of a 288-row region): the fp32 accumulators bit for bit."""
    announce(f"mxfp4_linear exact tile {tname} M={M} N={N} K={K}")
    Xq, Xs = exact_operands(M, K, 130 + M)
    Wq, Ws = exact_operands(N, K, 140 + N)
    _, acc = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, want_acc=True)
    Y = to_host(qdt.mxfp4_linear(to_dev(Xq), ex_dev(Xs), to_dev(Wq), ex_dev(Ws), None, "acc_f32", tile=tile))
    assert np.array_equal(Y.astype(np.float64), acc), f"{np.sum(Y != acc)} accumulators differ"


@pytest.mark.parametrize("M,F,K", [(300, 272, 512), (600, 384, 1024)])
def test_mxfp4_288x256_epilogues_exact_sums(M, F, K):
    """The 288 x 256 tile's fused epilogues on exact-sum inputs: bias bit for bit, gated SiLU and
    head RMSNorm within 1 ulp of the oracle."""
    announce(f"mxfp4_linear 288x256 epilogues M={M} F={F} K={K}")
    t = qdt.QDT_TILE_288x256
    Xq, Xs = exact_operands(M, K, 150 + M)
    Wq, Ws = exact_operands(2 * F, K, 160 + F)
    rng = np.random.default_rng(F)
    bias = W.f32_to_bf16_bits(rng.standard_normal(2 * F).astype(np.float32) * 4)
    dX, dXs, dW, dWs, db = to_dev(Xq), ex_dev(Xs), to_dev(Wq), ex_dev(Ws), to_dev(bias)
    Yb = to_host(qdt.mxfp4_linear(dX, dXs, dW, dWs, db, "bias", tile=t))
    assert bits_equal(Yb, oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias))
    Ys = to_host(qdt.mxfp4_linear(dX, dXs, dW, dWs, db, "silu_gate", tile=t))
    assert ulp_bf16(Ys, oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias, epi="silu_gate")).max() <= 1
    N = 512
    gamma = W.f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(256)).astype(np.float32))
    Yr = to_host(qdt.mxfp4_linear(dX, dXs, to_dev(Wq[:N]), ex_dev(Ws[:N]), to_dev(bias[:N]), "head_rmsnorm",
                                  gamma=to_dev(gamma), eps=1e-6, tile=t))
    Yr_ref = oracle.mxfp4_gemm_rows(Xq, Xs, Wq[:N], Ws[:N], bias[:N], epi="head_rmsnorm", gamma=gamma, eps=1e-6)
    assert ulp_bf16(Yr, Yr_ref).max() <= 1


def test_mxfp4_results_do_not_depend_on_tile():
    """General inputs, no K split: every output's K reduction runs through the same MFMA sequence
    whatever the tile, so the outputs of all FP4 tiles are identical bit for bit."""
    M, N, K = 600, 1024, 4608
    announce(f"mxfp4_linear tile independence M={M} N={N} K={K}")
    d = W.make_linear(M, N, K, seed=4400, x_kind="pct1", w_sigma=0.015, bias=True, epi="head_rmsnorm")
    Xq, Xs = qdt.mxfp4_quantize(to_dev(d["X"]))
    Wq, Ws = qdt.mxfp4_quantize(to_dev(d["W"]))
    b, g = to_dev(d["bias"]), to_dev(d["gamma"])
    for epi, tiles in (("bias", [t for t, _ in MX_TILES]), ("acc_f32", [t for t, _ in MX_TILES]),
                       ("silu_gate", [qdt.QDT_TILE_256, qdt.QDT_TILE_288x256]),
                       ("head_rmsnorm", [qdt.QDT_TILE_256, qdt.QDT_TILE_288x256])):
        kw = dict(gamma=g, eps=d["eps"]) if epi == "head_rmsnorm" else {}
        outs = [to_host(qdt.mxfp4_linear(Xq, Xs, Wq, Ws, b, epi, tile=t, split_k=1, **kw)) for t in tiles]
        for t, o in zip(tiles[1:], outs[1:]):
            assert bits_equal(o, outs[0]), f"{epi}: tile {t} differs from 256 x 256"


@pytest.mark.parametrize("tile,tname", MX_TILES[1:], ids=[t[1] for t in MX_TILES[1:]])
def test_mxfp4_split_k_exact_tiles(tile, tname):
    """K split on the 288-row tiles: exact sums, accumulators and bias output bit for bit."""
    M, N, K = 300, 576, 16384
    plan = qdt.mxfp4_linear_plan(M, N, K, tile=tile)
    assert plan["split_k"] > 1 and plan["tile_m"] == 288
    announce(f"mxfp4_linear split-K {plan['split_k']} tile {tname} M={M} N={N} K={K}")
    Xq, Xs = small_operands(M, K, 170)
    Wq, Ws = small_operands(N, K, 180)
    bias = W.f32_to_bf16_bits(np.random.default_rng(3).standard_normal(N).astype(np.float32))
    dX, dXs, dW, dWs = to_dev(Xq), ex_dev(Xs), to_dev(Wq), ex_dev(Ws)
    Y_ref, acc = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias, want_acc=True)
    Yacc = to_host(qdt.mxfp4_linear(dX, dXs, dW, dWs, None, "acc_f32", tile=tile))
    assert np.array_equal(Yacc.astype(np.float64), acc), f"{np.sum(Yacc != acc)} accumulators differ"
    assert bits_equal(to_host(qdt.mxfp4_linear(dX, dXs, dW, dWs, to_dev(bias), "bias", tile=tile)), Y_ref)
