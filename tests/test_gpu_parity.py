"""Parity of the HIP path (through the C ABI) with the CPU oracle, element by element.

Integer stages (calibration max-abs, lambda, inv_lambda, Wq, w_scale, Xq, x_scale, int32
accumulators) must be bit-exact; bf16 outputs within 1 bf16 ulp of the oracle (0 expected for
the BIAS epilogue, whose fp32 operation sequence is fixed on both sides).  Sizes here span
several tiles and ragged tails and finish on the oracle in seconds; the full workload sizes
are covered in test_gpu_workloads.py.
"""
import numpy as np
import pytest

import oracle
import qdt_workloads as W
from qdt_testutil import bits_equal, is_nan_bf16, to_dev, to_host, ulp_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
qdt = pytest.importorskip("quantized_diffusion_transformer_amd")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def prepared(d, smooth=True):
    """Oracle and device prepare + quantize for inputs d; returns (ref dict, dev dict)."""
    X, Wt = to_dev(d["X"]), to_dev(d["W"])
    s_ref = oracle.channel_absmax(d["X"]) if smooth else None
    Wq_r, sw_r, inv_r, lam_r = oracle.smooth_prepare(d["W"], s_ref)
    Xq_r, sx_r = oracle.quantize_per_token(d["X"], inv_r if smooth else None)
    s = qdt.channel_absmax(X) if smooth else None
    Wq, sw, inv, lam = qdt.smooth_prepare(Wt, s)
    Xq, sx = qdt.quantize_per_token(X, inv if smooth else None)
    torch.cuda.synchronize()
    ref = dict(s=s_ref, Wq=Wq_r, sw=sw_r, inv=inv_r, lam=lam_r, Xq=Xq_r, sx=sx_r)
    dev = dict(s=s, Wq=Wq, sw=sw, inv=inv, lam=lam, Xq=Xq, sx=sx, X=X, W=Wt)
    return ref, dev


def assert_stages_exact(ref, dev):
    for k in ("s", "Wq", "sw", "inv", "lam", "Xq", "sx"):
        if ref[k] is None:
            continue
        got = to_host(dev[k])
        assert bits_equal(got, ref[k]), f"{k}: {np.sum(got != ref[k])} elements differ"


# ------------------------------------------------------------------------------ quantize
@pytest.mark.parametrize("M,K,kind,zero_after", [
    (64, 256, "four20", None),
    (9, 1984, "pct1", None),        # one wave per row: 4, 6, 9, 12 and 16 chunks per lane
    (7, 2560, "four20", None),
    (600, 4608, "pct1", 590),       # ragged row count, 10 zero rows
    (13, 6080, "pareto", 11),
    (21, 8128, "pct1", None),       # 16 chunks per lane, the last lanes' last chunk absent
    (37, 12288, "pct1", None),      # 4 waves per row
    (1600, 12288, "pct1", 1500),    # 4 waves per row, blocks taking several rows (next row prefetched), zero rows
    (1000, 8256, "pareto", None),   # the same, ragged chunks
    (19, 53248, "pareto", 17),      # 16 waves per row (deep K), 7 chunks per lane
    (3, 57344, "pct1", None),       # the largest K with 7 chunks per lane
    (3, 57408, "pareto", None),     # the smallest with 16
    (3, 131072, "pct1", None),      # largest K
    (5, 64, "none", None),
])
def test_quantize_per_token_bit_exact(M, K, kind, zero_after):
    announce(f"quantize M={M} K={K}")
    X = W.activations(M, K, seed=77 + K, kind=kind, zero_rows_after=zero_after)
    inv = (2.0 ** np.random.default_rng(K).uniform(-3, 3, K)).astype(np.float32)
    for cm in (inv, None):
        q_r, s_r = oracle.quantize_per_token(X, cm)
        q, s = qdt.quantize_per_token(to_dev(X), None if cm is None else to_dev(cm))
        torch.cuda.synchronize()
        assert bits_equal(to_host(s), s_r)
        assert bits_equal(to_host(q), q_r), f"{np.sum(to_host(q) != q_r)} codes differ"


def test_quantize_row_stride_and_tiny_scales():
    announce("quantize strided + tiny scales")
    M, K, ld = 33, 1024, 1536
    rng = np.random.default_rng(3)
    big = W.f32_to_bf16_bits(rng.standard_normal((M, ld)).astype(np.float32))
    # rows at the bottom of the fp32 range: scale below FLT_MIN takes the division path
    big[5, :K] = W.f32_to_bf16_bits((rng.standard_normal(K) * 1e-37).astype(np.float32))
    big[6, :K] = W.f32_to_bf16_bits((rng.standard_normal(K) * 1e-39).astype(np.float32))
    big[7, :K] = 0
    big[8, :K] = W.f32_to_bf16_bits(np.float32([127.0, 2.5, 3.5, -2.5] + [0.5] * (K - 4)))
    Xd = to_dev(big)[:, :K]
    q, s = qdt.quantize_per_token(Xd, None)
    q_r, s_r = oracle.quantize_per_token(np.ascontiguousarray(big[:, :K]), None)
    torch.cuda.synchronize()
    assert bits_equal(to_host(s), s_r) and bits_equal(to_host(q), q_r)
    assert to_host(q)[8, :4].tolist() == [127, 2, 4, -2]


# ------------------------------------------------------------------------------ prepare
@pytest.mark.parametrize("N,K", [(128, 256), (4608, 4608), (300, 53248)])
def test_smooth_prepare_bit_exact(N, K):
    announce(f"prepare N={N} K={K}")
    d = W.make_linear(97, N, K, seed=5 + N, x_kind="pareto", w_sigma=0.015)
    ref, dev = prepared(d)
    assert_stages_exact(ref, dev)


def test_smooth_prepare_without_smoothing_and_accumulated_calibration():
    announce("prepare no smoothing / accumulate")
    d = W.make_linear(300, 256, 1024, seed=8, x_kind="pct1")
    ref, dev = prepared(d, smooth=False)
    assert_stages_exact(ref, dev)
    assert np.all(to_host(dev["lam"]) == 1) and np.all(to_host(dev["inv"]) == 1)
    X = to_dev(d["X"])
    s = qdt.channel_absmax(X[:100])
    s = qdt.channel_absmax(X[100:], s)
    torch.cuda.synchronize()
    assert bits_equal(to_host(s), oracle.channel_absmax(d["X"]))


def test_smooth_prepare_zero_channels_and_zero_weight_rows():
    # lambda = 1 where s_j = 0 or w_j = 0 (both, for one column); an all-zero weight row gets
    # scale 0 and codes 0, and its outputs are the bias exactly
    announce("prepare zero channels / zero weight rows")
    M, N, K = 300, 256, 1024
    d = W.make_linear(M, N, K, seed=23, x_kind="pct1")
    X, Wt = d["X"].copy(), d["W"].copy()
    zx, zw, zr = [3, 100, 517, 1023], [5, 100, 900], [7, 200, 255]
    X[:, zx] = 0
    Wt[:, zw] = 0
    Wt[zr, :] = 0
    d = dict(d, X=X, W=Wt)
    ref, dev = prepared(d)
    assert_stages_exact(ref, dev)
    lam, inv, sw, Wq = (to_host(dev[k]) for k in ("lam", "inv", "sw", "Wq"))
    for j in sorted(set(zx) | set(zw)):
        assert lam[j] == 1.0 and inv[j] == 1.0, j
    assert np.all(sw[zr] == 0) and np.all(Wq[zr] == 0)
    assert np.all(sw[np.setdiff1d(np.arange(N), zr)] > 0)
    b = to_dev(d["bias"])
    Y = qdt.w8a8_linear(dev["Xq"], dev["sx"], dev["Wq"], dev["sw"], b, "bias")
    torch.cuda.synchronize()
    Y = to_host(Y)
    Y_ref = oracle.epilogue(oracle.gemm_i32(ref["Xq"], ref["Wq"]), ref["sx"], ref["sw"], d["bias"], "bias")
    assert bits_equal(Y, Y_ref)
    assert np.all(Y[:, zr] == d["bias"][zr][None, :])


def test_smooth_prepare_other_alpha_close():
    # alpha != 0.5 uses powf on both sides; parity unpinned bit-wise (tolerance only)
    announce("prepare alpha 0.25")
    d = W.make_linear(64, 256, 512, seed=9, x_kind="four20")
    s_r = oracle.channel_absmax(d["X"])
    _, _, _, lam_r = oracle.smooth_prepare(d["W"], s_r, 0.25)
    _, _, _, lam = qdt.smooth_prepare(to_dev(d["W"]), to_dev(s_r), 0.25)
    torch.cuda.synchronize()
    assert np.allclose(to_host(lam), lam_r, rtol=4e-7, atol=0)


# ------------------------------------------------------------------------------ GEMM + epilogues
SHAPES = [
    (64, 128, 256),     # one partial tile
    (600, 1024, 1024),  # ragged M over 3 tile rows, several tile columns
    (289, 576, 640),    # just past one 288 tile; K = 5 stages
    (1, 16, 128),       # smallest legal problem
]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("tile,split", [(None, None), (qdt.QDT_TILE_256, 1), (qdt.QDT_TILE_288, 1),
                                        (qdt.QDT_TILE_288x256, 1), (qdt.QDT_TILE_256, 3),
                                        (qdt.QDT_TILE_288x256, 2), (qdt.QDT_TILE_224x256, 1),
                                        (qdt.QDT_TILE_224x256, 3)])
def test_int32_accumulators_bit_exact(M, N, K, tile, split):
    announce(f"acc M={M} N={N} K={K} tile={tile} split={split}")
    d = W.make_linear(M, N, K, seed=M + N + K, x_kind="pct1")
    ref, dev = prepared(d)
    acc = qdt.w8a8_linear(dev["Xq"], dev["sx"], dev["Wq"], dev["sw"], None, "acc_i32", tile=tile, split_k=split)
    torch.cuda.synchronize()
    want = oracle.gemm_i32(ref["Xq"], ref["Wq"])
    got = to_host(acc)
    assert np.array_equal(got, want), f"{np.sum(got != want)} accumulators differ"
    assert np.array_equal(want.astype(np.int64), oracle.gemm_i64(ref["Xq"], ref["Wq"]))


def test_int32_extreme_accumulators():
    # every product 127 * 127 (or -127 * 127) at the deepest K of the workloads
    announce("acc extremes K=53248")
    M, N, K = 40, 48, 53248
    Xq = np.full((M, K), 127, np.int8)
    Xq[1::2] = -127
    Wq = np.full((N, K), 127, np.int8)
    acc = qdt.w8a8_linear(to_dev(Xq), to_dev(np.ones(M, np.float32)), to_dev(Wq), to_dev(np.ones(N, np.float32)),
                          None, "acc_i32")
    torch.cuda.synchronize()
    got = to_host(acc).astype(np.int64)
    assert np.all(got[0::2] == 127 * 127 * K) and np.all(got[1::2] == -127 * 127 * K)


def run_linear(d, epi, tile=None, split=None, bias=True):
    ref, dev = prepared(d)
    b = to_dev(d["bias"]) if (bias and d.get("bias") is not None) else None
    kw = {}
    if epi == "head_rmsnorm":
        kw = dict(gamma=to_dev(d["gamma"]), eps=d["eps"])
    Y = qdt.w8a8_linear(dev["Xq"], dev["sx"], dev["Wq"], dev["sw"], b, epi, tile=tile, split_k=split, **kw)
    torch.cuda.synchronize()
    Y_ref = oracle.epilogue(oracle.gemm_i32(ref["Xq"], ref["Wq"]), ref["sx"], ref["sw"],
                            d["bias"] if b is not None else None, epi, d.get("gamma"), 256, d.get("eps", 1e-6))
    return to_host(Y), Y_ref, ref, dev


@pytest.mark.parametrize("M,N,K", SHAPES + [(700, 4608, 4608)])
@pytest.mark.parametrize("tile,split", [(None, None), (qdt.QDT_TILE_288, 1), (qdt.QDT_TILE_256, 4),
                                        (qdt.QDT_TILE_288x256, 1), (qdt.QDT_TILE_224x256, 1)])
def test_bias_epilogue_exact(M, N, K, tile, split):
    announce(f"bias M={M} N={N} K={K} tile={tile} split={split}")
    d = W.make_linear(M, N, K, seed=11 + M, x_kind="pct1")
    Y, Y_ref, _, _ = run_linear(d, "bias", tile, split)
    assert not is_nan_bf16(Y).any()
    u = ulp_bf16(Y, Y_ref)
    assert u.max() <= 1, f"max ulp {u.max()}"
    assert u.max() == 0, f"BIAS epilogue not bit-exact: {np.sum(u > 0)} elements at 1 ulp"


@pytest.mark.parametrize("M,F,K", [(64, 64, 256), (300, 640, 1024), (513, 1152, 512)])
@pytest.mark.parametrize("tile,split", [(None, None), (None, 3), (qdt.QDT_TILE_288x256, 1),
                                        (qdt.QDT_TILE_224x256, 1)])
def test_silu_gate_epilogue(M, F, K, tile, split):
    announce(f"silu M={M} F={F} K={K} tile={tile} split={split}")
    d = W.make_linear(M, 2 * F, K, seed=21 + M, x_kind="pct1", bias=True)
    Y, Y_ref, _, _ = run_linear(d, "silu_gate", tile=tile, split=split)
    assert Y.shape == (M, F) and not is_nan_bf16(Y).any()
    u = ulp_bf16(Y, Y_ref)
    assert u.max() <= 1, f"max ulp {u.max()}"


@pytest.mark.parametrize("split", [None, 2])
def test_silu_gate_large_gates(split):
    """Gate values far beyond |g| = 64 (where the exact expf / division form takes over): the
    sigmoid tail underflows to +-0 or tiny values exactly as in the oracle, within 1 ulp."""
    announce(f"silu large gates split={split}")
    M, F, K = 96, 128, 256
    d = W.make_linear(M, 2 * F, K, seed=77, x_kind="none", w_sigma=8.0, bias=True)
    Y, Y_ref, ref, _ = run_linear(d, "silu_gate", split=split)
    acc = oracle.gemm_i32(ref["Xq"], ref["Wq"]).astype(np.float64)
    g = acc[:, :F] * ref["sx"][:, None] * ref["sw"][None, :F]
    assert (np.abs(g) > 64).mean() > 0.2 and (np.abs(g) <= 64).mean() > 0.2  # both forms exercised
    assert not is_nan_bf16(Y).any()
    u = ulp_bf16(Y, Y_ref)
    assert u.max() <= 1, f"max ulp {u.max()}"


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (300, 1024, 1024), (257, 512, 4608)])
@pytest.mark.parametrize("tile,split", [(None, None), (None, 3), (qdt.QDT_TILE_288x256, 1),
                                        (qdt.QDT_TILE_224x256, 1), (qdt.QDT_TILE_224x256, 2)])
def test_head_rmsnorm_epilogue(M, N, K, tile, split):
    announce(f"rmsnorm M={M} N={N} K={K} tile={tile} split={split}")
    d = W.make_linear(M, N, K, seed=31 + M, x_kind="pct1", epi="head_rmsnorm")
    Y, Y_ref, _, _ = run_linear(d, "head_rmsnorm", tile=tile, split=split)
    assert not is_nan_bf16(Y).any()
    u = ulp_bf16(Y, Y_ref)
    assert u.max() <= 1, f"max ulp {u.max()}"


@pytest.mark.parametrize("epi", ["bias", "silu_gate", "head_rmsnorm", "acc_i32"])
@pytest.mark.parametrize("split", [None, 3])
def test_strided_output_into_wider_buffer(epi, split):
    """Y written into a column window of a wider row-major buffer (ldy > N_out): the window
    equals the packed result and the columns around it keep their sentinel."""
    announce(f"strided output epi={epi} split={split}")
    M, N, K = 300, 512, 1024
    d = W.make_linear(M, N, K, seed=57, x_kind="pct1", epi=epi if epi == "head_rmsnorm" else "bias")
    ref, dev = prepared(d)
    b = to_dev(d["bias"])
    kw = dict(gamma=to_dev(d["gamma"]), eps=d["eps"]) if epi == "head_rmsnorm" else {}
    nout = N // 2 if epi == "silu_gate" else N
    dt = torch.int32 if epi == "acc_i32" else torch.bfloat16
    packed = qdt.w8a8_linear(dev["Xq"], dev["sx"], dev["Wq"], dev["sw"], b, epi, split_k=split, **kw)
    wide = torch.full((M, nout + 48), 7, dtype=dt, device="cuda")
    view = wide[:, 16:16 + nout]
    qdt.w8a8_linear(dev["Xq"], dev["sx"], dev["Wq"], dev["sw"], b, epi, out=view, split_k=split, **kw)
    torch.cuda.synchronize()
    assert view.stride(0) == nout + 48
    assert torch.equal(view, packed)
    assert bool((wide[:, :16] == 7).all()) and bool((wide[:, 16 + nout:] == 7).all())


def test_results_do_not_depend_on_plan():
    # the integer sum is exact and every element gets the same fp32 sequence, so every plan
    # (tile shape, K split) gives the same bits; rows are independent of M
    announce("plan independence")
    d = W.make_linear(600, 1152, 2048, seed=41, x_kind="pct1")
    outs = [run_linear(d, "bias", t, s)[0] for t, s in ((None, None), (qdt.QDT_TILE_288, 1), (qdt.QDT_TILE_256, 1),
                                                         (qdt.QDT_TILE_256, 5), (qdt.QDT_TILE_288, 2),
                                                         (qdt.QDT_TILE_288x256, 1), (qdt.QDT_TILE_288x256, 3),
                                                         (qdt.QDT_TILE_224x256, 1))]
    for o in outs[1:]:
        assert bits_equal(o, outs[0])
    ref, dev = prepared(d)
    b = to_dev(d["bias"])
    sub = qdt.w8a8_linear(dev["Xq"][:37], dev["sx"][:37], dev["Wq"], dev["sw"], b, "bias")
    torch.cuda.synchronize()
    assert bits_equal(to_host(sub), outs[0][:37])


@pytest.mark.parametrize("epi", ["head_rmsnorm", "silu_gate"])
def test_fused_epilogues_do_not_depend_on_plan(epi):
    # the gated SiLU and the head RMSNorm give the same bits under every tile and K split: the
    # split-K epilogue sums a head's squares in the fused kernel's order
    announce(f"plan independence {epi}")
    d = W.make_linear(600, 1024, 2048, seed=43, x_kind="pct1", epi=epi)
    outs = [run_linear(d, epi, t, s)[0] for t, s in ((None, None), (qdt.QDT_TILE_256, 1), (qdt.QDT_TILE_256, 3),
                                                     (qdt.QDT_TILE_256, 7), (qdt.QDT_TILE_288x256, 1),
                                                     (qdt.QDT_TILE_288x256, 2), (qdt.QDT_TILE_224x256, 1),
                                                     (qdt.QDT_TILE_224x256, 3))]
    for o in outs[1:]:
        assert bits_equal(o, outs[0]), f"{np.sum(o != outs[0])} elements differ between plans"


def test_zero_rows_give_bias_and_padding_keeps_rows():
    # the zero-padded text projection: zero rows project to the bias, real rows unchanged
    announce("zero rows / padding")
    M, N, K, T = 700, 512, 2048, 120
    pad = W.make_linear(M, N, K, seed=51, x_kind="pareto", zero_rows_after=T)
    real = W.make_linear(T, N, K, seed=51, x_kind="pareto")
    Yp, Yp_ref, _, _ = run_linear(pad, "bias")
    Yr, _, _, _ = run_linear(real, "bias")
    assert np.array_equal(W.bf16_bits_to_f32(Yp[T:]), np.broadcast_to(W.bf16_bits_to_f32(pad["bias"]), (M - T, N)))
    assert bits_equal(Yp[:T], Yr)
    assert ulp_bf16(Yp, Yp_ref).max() == 0


def test_bias_none_and_empty_rows():
    announce("no bias / M=0")
    d = W.make_linear(70, 256, 512, seed=61, x_kind="pct1")
    Y, Y_ref, _, _ = run_linear(d, "bias", bias=False)
    assert ulp_bf16(Y, Y_ref).max() == 0
    ref, dev = prepared(d)
    out = qdt.w8a8_linear(dev["Xq"][:0], dev["sx"][:0], dev["Wq"], dev["sw"], None, "bias")
    assert out.shape == (0, 256)


# ------------------------------------------------------------------------------ bf16 linear
def bf16_bound_check(Z, H, Wd, bias, rows=None):
    """|Z - Z_ref| <= ulp_bf16(Z_ref) + gamma_K sum_k |h_k w_k|, with Z_ref the fp64 product."""
    Hf = W.bf16_bits_to_f32(H if rows is None else H[rows]).astype(np.float64)
    Wf = W.bf16_bits_to_f32(Wd).astype(np.float64)
    ref = Hf @ Wf.T
    if bias is not None:
        ref += W.bf16_bits_to_f32(bias).astype(np.float64)[None, :]
    K = H.shape[1]
    u = 2.0 ** -24
    gam = K * u / (1 - K * u)
    bound = gam * (np.abs(Hf) @ np.abs(Wf).T)
    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126)))
    ulp = 2.0 ** (e - 7)
    Zf = W.bf16_bits_to_f32(Z).astype(np.float64)
    err = np.abs(Zf - ref)
    assert np.all(err <= ulp + bound), f"max excess {np.max(err - ulp - bound)}"
    oz = oracle.bf16_gemm_rows(H, Wd, bias, rows)
    return ulp_bf16(Z, oz)


@pytest.mark.parametrize("M,N,K", [(64, 128, 256), (600, 1024, 2048), (290, 576, 12288)])
def test_bf16_linear_within_bound(M, N, K):
    announce(f"bf16 M={M} N={N} K={K}")
    rng = np.random.default_rng(M)
    H = W.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    Wd = W.f32_to_bf16_bits((0.01 * rng.standard_normal((N, K))).astype(np.float32))
    bias = W.f32_to_bf16_bits((0.01 * rng.standard_normal(N)).astype(np.float32))
    for b in (bias, None):
        Z = qdt.bf16_linear(to_dev(H), to_dev(Wd), None if b is None else to_dev(b))
        torch.cuda.synchronize()
        u = bf16_bound_check(to_host(Z), H, Wd, b)
        # the bound is the gate; near cancellation it allows many ulps, elsewhere expect <= 1
        assert np.mean(u <= 1) > 0.99
