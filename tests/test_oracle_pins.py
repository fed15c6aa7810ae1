"""Pins of the CPU oracle against facts other than itself (no GPU).

Each test checks the oracle against a closed form, an invariant of the method, a
special case that reduces to a library routine, brute force on tiny inputs, or a
number printed on the pages -- chosen so that a plausible mistake (a dropped term,
a wrong sign or index, a transposed operand, a wrong rounding rule) fails one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import qdt_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


def f32(b):
    return W.bf16_bits_to_f32(b)


def ulp_dist_bf16(a, b):
    """Distance in bf16 ulps between bit patterns, via the order-preserving integer map."""
    def key(u):
        u = np.asarray(u, np.int32)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + (u & 0x7FFF))
    return np.abs(key(a) - key(b))


# ----------------------------------------------------------------------------- bf16 rounding
def test_bf16_round_half_even_ties():
    one = 1.0
    cases = {
        one + 2.0 ** -8: one,                          # tie, even neighbour is 1.0
        one + 2.0 ** -7 + 2.0 ** -8: one + 2.0 ** -6,  # tie, odd below -> rounds up to even
        one + 2.0 ** -8 + 2.0 ** -20: one + 2.0 ** -7,  # just above the tie
        -(one + 2.0 ** -8): -one,
        3.0 * 2.0 ** -132: 3.0 * 2.0 ** -132,          # bf16 subnormal (multiple of 2^-133), exact
        2.0 ** -135: 0.0,                              # below half the smallest bf16 subnormal
    }
    for x, want in cases.items():
        got = f32(oracle.f32_to_bf16(np.float32(x)))[0]
        assert got == np.float32(want), (x, got, want)


def test_bf16_rounding_matches_torch_cpu():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        (rng.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32)
                         & np.uint32(0x7F7FFFFF)).view(np.float32)])
    ours = oracle.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ----------------------------------------------------------------------------- integer GEMM
@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (3, 5, 64), (7, 2, 128), (8, 8, 256), (17, 33, 320)])
def test_gemm_equals_int64_matmul(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    A = rng.integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
    B = rng.integers(-127, 128, (N, K), dtype=np.int64).astype(np.int8)
    A[0, :] = 127
    B[-1, :] = -127
    ref = A.astype(np.int64) @ B.astype(np.int64).T
    assert np.array_equal(oracle.gemm_i64(A, B), ref)
    assert np.array_equal(oracle.gemm_i32(A, B).astype(np.int64), ref)


@pytest.mark.parametrize("K", [4608, 53248])
def test_gemm_int32_extremes_no_overflow(K):
    # |acc| <= 127^2 K stays below 2^31 up to K = 133144; the extreme is reached here
    A = np.full((2, K), 127, np.int8)
    A[1] = -127
    B = np.full((3, K), 127, np.int8)
    B[2, ::2] = -127
    c32 = oracle.gemm_i32(A, B)
    c64 = oracle.gemm_i64(A, B)
    assert np.array_equal(c32.astype(np.int64), c64)
    assert c64[0, 0] == 127 * 127 * K and c64[1, 0] == -127 * 127 * K
    assert c64[0, 2] == 0


# ----------------------------------------------------------------------------- quantization
def test_quantize_round_half_even_on_exact_scale():
    # with no smoothing and a row maximum of 127 (exact in bf16) the scale is exactly 1.0,
    # so v / scale = v and the ties expose the rounding rule
    row = np.array([127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 126.5, -0.5, 0.25, -1.5, 5.5] + [0.0] * 52, np.float32)
    q, s = oracle.quantize_rows(bf(row[None, :]))
    assert s[0] == np.float32(1.0)
    want = [127, 2, 4, -2, -4, 0, 2, 126, 0, 0, -2, 6]
    assert q[0, :12].tolist() == want


def _quant_bounds(X, colmul, q, s):
    x = f32(X).astype(np.float32)
    v = (x * colmul[None, :]).astype(np.float32) if colmul is not None else x
    v64 = v.astype(np.float64)
    amax = np.abs(v64).max(axis=1)
    nz = amax > 0
    # zero rows: zero scale and codes
    assert np.all(s[~nz] == 0) and np.all(q[~nz] == 0)
    # scale is amax/127 to within one fp32 rounding
    assert np.all(np.abs(s[nz].astype(np.float64) * 127.0 - amax[nz]) <= amax[nz] * 2.0 ** -23)
    # every nonzero row uses the full symmetric range, never -128
    assert np.all(np.abs(q[nz].astype(np.int32)).max(axis=1) == 127)
    assert q.min() >= -127
    # reconstruction error of round-to-nearest: |v - q s| <= s/2 (1 + 2^-15)
    err = np.abs(v64 - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * 0.5 * (1.0 + 2.0 ** -15))


@pytest.mark.parametrize("seed", range(12))
def test_quantize_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, 9))
    K = int(rng.choice([64, 128, 256]))
    X = bf(rng.standard_normal((M, K)).astype(np.float32) * np.float32(10.0 ** rng.uniform(-3, 3)))
    X[rng.integers(0, M)] = 0  # one all-zero row
    colmul = (2.0 ** rng.uniform(-4, 4, K)).astype(np.float32)
    for cm in (None, colmul):
        q, s = oracle.quantize_rows(X, cm)
        _quant_bounds(X, cm, q, s)
        # every code is the nearest integer to v/s computed in fp64 except at (near-)ties
        x = f32(X)
        v = (x * cm[None, :]).astype(np.float32) if cm is not None else x
        nz = s > 0
        t = v[nz].astype(np.float64) / s[nz, None].astype(np.float64)
        near_tie = np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-4
        assert np.all((q[nz] == np.round(t)) | near_tie)


@pytest.mark.parametrize("k", [-3, 1, 5])
def test_quantize_power_of_two_invariance(k):
    d = W.make_linear(16, 8, 256, seed=7, x_kind="four20")
    q0, s0 = oracle.quantize_rows(d["X"])
    Xs = bf(f32(d["X"]) * np.float32(2.0 ** k))  # exact scaling by 2^k
    q1, s1 = oracle.quantize_rows(Xs)
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, (s0 * np.float32(2.0 ** k)).astype(np.float32))


def test_per_token_scales_are_per_row():
    # rows of very different magnitude each get their own scale (a per-tensor scale fails)
    X = bf(np.outer(10.0 ** np.arange(-4, 4), np.linspace(-1, 1, 64)).astype(np.float32))
    q, s = oracle.quantize_rows(X)
    assert np.all(np.abs(q).max(axis=1) == 127)
    assert np.all(np.diff(np.log10(s)) > 0.9)


# ----------------------------------------------------------------------------- smoothing
def test_lambda_closed_form_on_powers_of_four():
    a = np.arange(-6, 7)
    b = np.arange(6, -7, -1)
    s = (4.0 ** a).astype(np.float32)
    w = (4.0 ** b).astype(np.float32)
    lam, inv = oracle.smooth_lambda(s, w, 0.5)
    assert np.array_equal(lam, (2.0 ** (a - b)).astype(np.float32))
    assert np.array_equal(inv, (2.0 ** (b - a)).astype(np.float32))


def test_lambda_zero_channels_and_other_alpha():
    s = np.array([0.0, 3.0, 0.0, 2.0], np.float32)
    w = np.array([1.0, 0.0, 0.0, 0.5], np.float32)
    lam, inv = oracle.smooth_lambda(s, w, 0.5)
    assert lam[:3].tolist() == [1.0, 1.0, 1.0] and inv[:3].tolist() == [1.0, 1.0, 1.0]
    assert lam[3] == np.float32(2.0)
    # alpha = 1 moves everything into the weights: lambda = s; alpha = 0: lambda = 1/w
    lam1, _ = oracle.smooth_lambda(s[3:], w[3:], 1.0)
    lam0, _ = oracle.smooth_lambda(s[3:], w[3:], 0.0)
    assert lam1[0] == np.float32(2.0) and lam0[0] == np.float32(2.0)
    lamq, _ = oracle.smooth_lambda(np.float32([16.0]), np.float32([81.0]), 0.25)
    assert abs(float(lamq[0]) - 2.0 / 27.0) < 1e-6


def test_smoothing_balances_channel_ranges():
    # with alpha = 0.5 the smoothed activation and the smoothed weight of channel j
    # share the same max-abs, sqrt(s_j w_j)
    d = W.make_linear(64, 96, 256, seed=11, x_kind="four20")
    s = oracle.channel_absmax(d["X"])
    Wq, sw, inv, lam = oracle.smooth_prepare(d["W"], s, 0.5)
    x = f32(d["X"]).astype(np.float64)
    w = f32(d["W"]).astype(np.float64)
    xs = np.abs(x * inv[None, :]).max(axis=0)
    ws = np.abs(w * lam[None, :]).max(axis=0)
    target = np.sqrt(s.astype(np.float64) * np.abs(w).max(axis=0))
    assert np.allclose(xs, target, rtol=4e-7) and np.allclose(ws, target, rtol=4e-7)
    assert np.all(np.abs(inv.astype(np.float64) * lam.astype(np.float64) - 1.0) <= 2.0 ** -23)


def test_channel_absmax_accumulates():
    d = W.make_linear(40, 8, 128, seed=3, x_kind="four20")
    full = oracle.channel_absmax(d["X"])
    part = oracle.channel_absmax(d["X"][:13])
    acc = oracle.channel_absmax(d["X"][13:], part)
    assert np.array_equal(full, acc)
    assert np.array_equal(full, np.abs(f32(d["X"])).max(axis=0))


def _reconstruction_bound_check(r, X, Wt):
    """sum_j (qx sx)(qw sw) reproduces X W^T within the quantization and rounding bound."""
    x = f32(X).astype(np.float64)
    w = f32(Wt).astype(np.float64)
    sx = r["sx"].astype(np.float64)
    sw = r["sw"].astype(np.float64)
    xh = r["Xq"].astype(np.float64) * sx[:, None]
    wh = r["Wq"].astype(np.float64) * sw[:, None]
    approx = xh @ wh.T
    exact = x @ w.T
    xs = np.abs(x * r["inv_lambda"][None, :].astype(np.float64))
    ws = np.abs(w * r["lam"][None, :].astype(np.float64))
    h = 0.5 * (1.0 + 2.0 ** -15)
    bound = (h * xs @ np.ones_like(ws).T * sw[None, :] + h * np.ones_like(xs) @ ws.T * sx[:, None]
             + h * h * X.shape[1] * sx[:, None] * sw[None, :] + 4 * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T))
    assert np.all(np.abs(approx - exact) <= bound)
    return approx, exact


def test_smoothquant_invariant_through_quantization():
    # X diag(lambda)^-1 diag(lambda) W = X W: the dequantized product must approximate the
    # unsmoothed product; applying lambda on the wrong side (or twice) breaks the bound.
    d = W.make_linear(24, 40, 512, seed=21, x_kind="four20", w_sigma=0.02)
    r = oracle.linear(d["X"], d["W"], d["bias"])
    _reconstruction_bound_check(r, d["X"], d["W"])
    # planted mistake: lambda applied to the activations instead of its inverse
    bad = dict(r)
    bad["Xq"], bad["sx"] = oracle.quantize_rows(d["X"], r["lam"])
    with pytest.raises(AssertionError):
        _reconstruction_bound_check(bad, d["X"], d["W"])


def test_smoothquant_exact_with_power_of_two_lambda():
    # columns whose calibration max and weight max are powers of 4 give lambda = 2^k:
    # then x_hat * w_hat == x * w exactly for every product, so X_hat W_hat^T == X W^T in fp64
    rng = np.random.default_rng(4)
    M, N, K = 6, 5, 64
    x = (0.5 * rng.standard_normal((M, K))).astype(np.float32)   # |x| < 4 in practice
    w = (0.01 * rng.standard_normal((N, K))).astype(np.float32)  # |w| < 0.25 in practice
    X = bf(x); Wt = bf(w)
    xa = np.abs(f32(X)); wa = np.abs(f32(Wt))
    ia = xa.argmax(axis=0); iw = wa.argmax(axis=0)
    X[ia, np.arange(K)] = bf(np.sign(f32(X[ia, np.arange(K)])) * 4.0 ** rng.integers(1, 3, K))
    Wt[iw, np.arange(K)] = bf(np.sign(f32(Wt[iw, np.arange(K)])) * 4.0 ** rng.integers(-1, 1, K))
    s = oracle.channel_absmax(X)
    assert np.all(np.log2(s) % 2 == 0)
    _, _, inv, lam = oracle.smooth_prepare(Wt, s, 0.5)
    assert np.all(np.log2(lam) == np.round(np.log2(lam)))
    xh = (f32(X) * inv[None, :]).astype(np.float64)
    wh = (f32(Wt) * lam[None, :]).astype(np.float64)
    assert np.array_equal(xh @ wh.T, f32(X).astype(np.float64) @ f32(Wt).astype(np.float64).T)


# ----------------------------------------------------------------------------- epilogues
def test_bias_epilogue_matches_fp64_dequant():
    rng = np.random.default_rng(9)
    M, N = 7, 19
    acc = rng.integers(-2 ** 24, 2 ** 24, (M, N)).astype(np.int32)
    acc[0, :5] = [0, 1, -1, 2 ** 30, -(2 ** 30)]
    sx = (rng.uniform(0.5, 2.0, M) * 1e-3).astype(np.float32)
    sw = (rng.uniform(0.5, 2.0, N) * 1e-4).astype(np.float32)
    bias = bf(rng.standard_normal(N) * 0.01)
    Y = oracle.epilogue(acc, sx, sw, bias, "bias")
    ref = acc.astype(np.float64) * sx[:, None].astype(np.float64) * sw[None, :].astype(np.float64) \
        + f32(bias).astype(np.float64)[None, :]
    refb = oracle.f32_to_bf16(ref.astype(np.float32).ravel()).reshape(M, N)
    assert ulp_dist_bf16(Y, refb).max() <= 1
    # transposed scales (sw per row) or a dropped bias is caught
    assert ulp_dist_bf16(oracle.epilogue(acc, sx, sw, None, "bias"), refb).max() > 1


def test_zero_rows_project_to_bias_exactly():
    # a zero row projects to the bias vector; rows are independent
    # (Faster Ideogram 4 with Less Prompt Compute, "Most of the Tensor Was Zero")
    d = W.make_linear(32, 48, 256, seed=5, x_kind="pareto", zero_rows_after=20)
    r = oracle.linear(d["X"], d["W"], d["bias"])
    assert np.all(r["sx"][20:] == 0) and np.all(r["Xq"][20:] == 0)
    assert np.array_equal(f32(r["Y"][20:]), np.broadcast_to(f32(d["bias"]), (12, 48)))


def test_rows_are_independent():
    d = W.make_linear(40, 64, 256, seed=6, x_kind="four20")
    r = oracle.linear(d["X"], d["W"], d["bias"])
    rows = np.array([39, 0, 17, 17, 5])
    Y = oracle.linear_rows(r["Xq"], r["sx"], r["Wq"], r["sw"], d["bias"], rows)
    assert np.array_equal(Y, r["Y"][rows])
    # padding with repeated rows (no new column maxima) leaves the real rows unchanged
    Xp = np.concatenate([d["X"], d["X"][::-1]], axis=0)
    rp = oracle.linear(Xp, d["W"], d["bias"], s=r["s"])
    assert np.array_equal(rp["Y"][:40], r["Y"])


def test_silu_gate_epilogue():
    from scipy.special import expit
    rng = np.random.default_rng(12)
    M, F = 5, 33
    acc = rng.integers(-3000, 3000, (M, 2 * F)).astype(np.int32)
    acc[:, 0] = 0          # g = 0 (with zero bias) -> 0
    acc[:, F + 1] = 0      # u = 0 -> 0
    sx = np.full(M, 1e-2, np.float32)
    sw = np.full(2 * F, 1e-2, np.float32)
    Y = f32(oracle.epilogue(acc, sx, sw, None, "silu_gate"))
    assert Y.shape == (M, F)
    assert np.all(Y[:, 0] == 0) and np.all(Y[:, 1] == 0)
    g = acc[:, :F].astype(np.float64) * 1e-4
    u = acc[:, F:].astype(np.float64) * 1e-4
    ref = g * expit(g) * u
    refb = f32(oracle.f32_to_bf16(ref.astype(np.float32).ravel()).reshape(M, F))
    assert ulp_dist_bf16(bf(Y), bf(refb)).max() <= 1
    # the gate/up roles are not symmetric: swapping them is caught
    swapped = u * expit(u) * g
    assert np.abs(swapped - Y).max() > 1e-3


def test_head_rmsnorm_closed_forms():
    hd = 256
    M, H = 4, 3
    N = hd * H
    rng = np.random.default_rng(13)
    gamma = bf(1.0 + 0.1 * rng.standard_normal(hd))
    g = f32(gamma).astype(np.float64)
    sx = np.ones(M, np.float32)
    sw = np.ones(N, np.float32)
    # head 0 constant c per row, head 1 random, head 2 random at 1000x the scale
    acc = np.zeros((M, N), np.int32)
    c = np.array([3, -7, 1, 100])
    acc[:, :hd] = c[:, None]
    acc[:, hd:2 * hd] = rng.integers(-50, 50, (M, hd))
    acc[:, 2 * hd:] = rng.integers(-50000, 50000, (M, hd))
    for eps in (1e-6, 1e-2):
        Y = f32(oracle.epilogue(acc, sx, sw, None, "head_rmsnorm", bf(f32(gamma)), hd, eps)).astype(np.float64)
        # constant head: y r gamma = gamma c / sqrt(c^2 + eps)
        want = g[None, :] * c[:, None] / np.sqrt(c[:, None].astype(np.float64) ** 2 + eps)
        assert np.all(np.abs(Y[:, :hd] - want) <= np.abs(want) * 2.0 ** -7)
        # each head is normalised on its own: sum (Y/gamma)^2 = hd * ms / (ms + eps)
        for h in (1, 2):
            y = acc[:, h * hd:(h + 1) * hd].astype(np.float64)
            ms = (y ** 2).mean(axis=1)
            lhs = ((Y[:, h * hd:(h + 1) * hd] / g[None, :]) ** 2).sum(axis=1)
            assert np.allclose(lhs, hd * ms / (ms + eps), rtol=2e-2)
    # tiny values: eps dominates, Y = y gamma / sqrt(eps)
    acc2 = np.ones((1, hd), np.int32)
    Y2 = f32(oracle.epilogue(acc2, np.float32([1e-6]), np.ones(hd, np.float32), None, "head_rmsnorm",
                             gamma, hd, 1e-2)).astype(np.float64)
    assert np.allclose(Y2[0], g * 1e-6 / np.sqrt(1e-2 + 1e-12), rtol=2 ** -7)


# ----------------------------------------------------------------------------- adaLN producer
def _ln_fp64(x, shift, scale, eps):
    """LayerNorm over each row in fp64 (biased variance), then x (1 + scale) + shift."""
    x = f32(x).astype(np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    n = (x - mu) / np.sqrt(var + eps)
    sc = 0.0 if scale is None else f32(scale).astype(np.float64)
    sh = 0.0 if shift is None else f32(shift).astype(np.float64)
    return n * (1.0 + sc) + sh


@pytest.mark.parametrize("K", [16, 256, 4608])
def test_adaln_matches_fp64_layernorm(K):
    rng = np.random.default_rng(20 + K)
    M = 12
    x = rng.standard_normal((M, K))
    x[:, rng.integers(0, K, max(1, K // 100))] *= 30.0          # outlier channels
    x[3] *= 1e-3                                                  # variance ~ eps: eps must count
    x[4] += 7.0                                                   # mean far from 0
    x[5] = np.abs(x[5])                                           # one-signed row
    X = bf(x)
    shift, scale = bf(0.3 * rng.standard_normal(K)), bf(0.5 * rng.standard_normal(K))
    for sh, sc in ((shift, scale), (None, None), (shift, None), (None, scale)):
        H = oracle.adaln_modulate(X, sh, sc, 1e-6)
        ref = _ln_fp64(X, sh, sc, 1e-6)
        # fp32 intermediates cost far less than half a bf16 ulp; the final rounding at most half an ulp
        assert np.all(ulp_dist_bf16(H, bf(ref)) <= 1)
        # the reference itself rounds to H on almost every element (not a 1-ulp drift everywhere)
        assert np.mean(ulp_dist_bf16(H, bf(ref)) == 0) > 0.99


def test_adaln_constant_rows_give_shift_exactly():
    K = 64
    rng = np.random.default_rng(21)
    X = bf(np.repeat(np.array([[0.0], [3.25], [-1e4], [1e-20]]), K, axis=1))
    shift, scale = bf(rng.standard_normal(K)), bf(rng.standard_normal(K))
    H = oracle.adaln_modulate(X, shift, scale, 1e-6)
    assert np.array_equal(H, np.broadcast_to(shift, H.shape))    # x - mean == 0 exactly
    H0 = oracle.adaln_modulate(X, None, scale, 1e-6)
    assert not f32(H0).any()


@pytest.mark.parametrize("k", [-6, 3])
def test_adaln_power_of_two_scaling_invariance(k):
    """With eps = 0 every step scales exactly by 2^k, so LayerNorm(2^k x) == LayerNorm(x) bit for bit."""
    rng = np.random.default_rng(22)
    X = bf(rng.standard_normal((6, 512)) * 4)
    X2 = bf(f32(X).astype(np.float64) * 2.0 ** k)
    assert np.array_equal(f32(X2).astype(np.float64), f32(X).astype(np.float64) * 2.0 ** k)
    shift, scale = bf(rng.standard_normal(512)), bf(rng.standard_normal(512))
    assert np.array_equal(oracle.adaln_modulate(X, shift, scale, 0.0), oracle.adaln_modulate(X2, shift, scale, 0.0))


def test_adaln_quantize_is_the_quantizer_on_h():
    """The fused producer's int8 codes are the per-token quantizer applied to H: checked here on
    H with a power-of-two row maximum, where the scale is exact and the codes are known."""
    K = 256
    X = np.zeros((2, K))
    X[:, 0], X[:, 1] = 1.0, -1.0          # mean 0, var 2/K: n = +-sqrt(K/2) = +-11.3137...
    shift = bf(np.zeros(K))
    scale = bf(np.zeros(K))
    Xq, sx, H = oracle.adaln_quantize(bf(X), shift, scale, None, 0.0)
    n = f32(H)
    assert n[0, 0] == -n[0, 1] and abs(n[0, 0] - math.sqrt(K / 2)) <= math.sqrt(K / 2) * 2.0 ** -8
    assert np.all(n[:, 2:] == 0)
    assert np.all(Xq[:, 0] == 127) and np.all(Xq[:, 1] == -127) and not Xq[:, 2:].any()
    assert np.all(sx == np.float32(n[0, 0]) / np.float32(127.0))


# ----------------------------------------------------------------------------- block-scaled FP4
FP4_POS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # the 2-bit-exponent, 1-bit-mantissa magnitudes


def test_fp4_code_table():
    vals = [oracle.fp4_value(c) for c in range(16)]
    assert vals[:8] == FP4_POS
    assert all(vals[8 + i] == -vals[i] for i in range(8))
    # one binade per exponent step: the spacing doubles from [1, 2) to [2, 4) to [4, 8)
    assert np.diff(FP4_POS[2:4]) == 0.5 and np.diff(FP4_POS[4:6]) == 1.0 and np.diff(FP4_POS[6:8]) == 2.0


def _mx_block(vals):
    """One 32-element bf16 row from up to 32 values (rest zero)."""
    v = np.zeros(32, np.float32)
    v[:len(vals)] = vals
    return bf(v)[None, :]


def test_mx_scale_rule_and_zero_blocks():
    rng = np.random.default_rng(30)
    x = rng.standard_normal((16, 256)) * 10.0 ** rng.integers(-6, 6, (16, 1))
    x[3, 64:96] = 0.0                                        # an all-zero block
    X = bf(x)
    Q, S = oracle.mxfp4_quantize(X)
    v = f32(X).astype(np.float64).reshape(16, 8, 32)
    amax = np.abs(v).max(axis=2)
    e = S.astype(np.int64) - 127
    nz = amax > 0
    ratio = amax[nz] / np.ldexp(1.0, e[nz])
    assert np.all((ratio >= 4.0) & (ratio < 8.0))            # the block max lands in [4, 8)
    assert S[3, 2] == 0 and not Q[3, 32:48].any()             # zero block: exponent -127, codes +0


def test_mx_rounding_nearest_ties_even_and_saturation():
    # block max 4 pins the exponent to 0 (scale 1), so every element is rounded as written
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    sat = {6.5: 6.0, 7.75: 6.0}
    t = list(ties) + list(sat) + [-0.25, -0.1, -5.0, 0.3, 0.7, 2.75, 4.5]
    want = list(ties.values()) + list(sat.values()) + [0.0, 0.0, -4.0, 0.5, 0.5, 3.0, 4.0]
    Q, S = oracle.mxfp4_quantize(_mx_block([4.0] + t))
    assert S[0, 0] == 127
    d = oracle.mxfp4_dequantize(Q, S)[0]
    assert list(d[1:1 + len(t)]) == want
    # negative values rounding to zero are stored as +0 (code 0)
    j = 1 + len(ties) + len(sat)                                 # the -0.25 element
    assert (Q[0, j // 2] >> (4 * (j % 2))) & 15 == 0
    # dense check: the decoded value is a nearest representable value
    rng = np.random.default_rng(31)
    vals = np.sort(rng.uniform(-6, 6, 31).astype(np.float32))
    Q, S = oracle.mxfp4_quantize(_mx_block(np.concatenate([[6.0], vals])))
    d = oracle.mxfp4_dequantize(Q, S)[0][1:]
    x = f32(bf(vals)).astype(np.float64)
    grid = np.array(FP4_POS + [-v for v in FP4_POS[1:]])
    best = np.abs(x[:, None] - grid[None, :]).min(axis=1)
    assert np.all(np.abs(x - d) == best)


def test_mx_nibble_order_and_lossless_values():
    codes = np.arange(32) % 16
    vals = np.array([oracle.fp4_value(c) for c in codes]) * 0.25   # block max 6 * 0.25 = 1.5 -> exponent -2
    Q, S = oracle.mxfp4_quantize(_mx_block(vals))
    assert S[0, 0] == 127 - 2
    assert Q[0, 0] == (codes[0] | (codes[1] << 4)) and Q[0, 5] == (codes[10] | (codes[11] << 4))
    assert np.array_equal(oracle.mxfp4_dequantize(Q, S)[0], vals)


def test_mx_error_bound():
    rng = np.random.default_rng(32)
    X = bf(rng.standard_normal((8, 512)) * 3)
    Q, S = oracle.mxfp4_quantize(X)
    x = f32(X).astype(np.float64)
    err = np.abs(oracle.mxfp4_dequantize(Q, S) - x)
    unit = np.repeat(np.ldexp(1.0, S.astype(np.int64) - 127), 32, axis=1)
    t = np.abs(x) / unit
    # half the grid spacing inside [0, 6]; up to the distance to 6 above it
    half = np.where(t < 2, 0.25, np.where(t < 4, 0.5, 1.0))
    assert np.all(np.where(t <= 6, err <= half * unit, err <= (t - 6) * unit + 1e-300))


def test_mx_column_multiplier_is_applied_first():
    """Power-of-two multipliers are exact, so quantizing X * colmul equals quantizing the scaled X."""
    rng = np.random.default_rng(34)
    X = bf(rng.standard_normal((4, 128)))
    mul = np.ldexp(1.0, rng.integers(-3, 4, 128)).astype(np.float32)
    Xm = bf(f32(X) * mul)
    assert np.array_equal(f32(Xm), f32(X) * mul)
    for a, b in zip(oracle.mxfp4_quantize(X, mul), oracle.mxfp4_quantize(Xm)):
        assert np.array_equal(a, b)
    assert not np.array_equal(oracle.mxfp4_quantize(X, mul)[0], oracle.mxfp4_quantize(X)[0])


def test_mx_head_rmsnorm_normalizes_each_head():
    rng = np.random.default_rng(35)
    M, N, K = 3, 512, 256
    Xq, Xs = oracle.mxfp4_quantize(bf(rng.standard_normal((M, K))))
    Wq, Ws = oracle.mxfp4_quantize(bf(rng.standard_normal((N, K)) * 0.05))
    gamma = bf(1.0 + 0.1 * rng.standard_normal(256))
    bias = bf(0.01 * rng.standard_normal(N))
    Y, acc = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias, want_acc=True, epi="head_rmsnorm", gamma=gamma, eps=1e-6)
    g = f32(gamma).astype(np.float64)
    y = acc + f32(bias).astype(np.float64)
    for h in range(N // 256):
        yh = y[:, h * 256:(h + 1) * 256]
        want = yh / np.sqrt((yh ** 2).mean(axis=1, keepdims=True) + 1e-6) * g
        got = f32(Y[:, h * 256:(h + 1) * 256]).astype(np.float64)
        assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 1e-30)


def test_mx_gemm_exact_against_rationals():
    from fractions import Fraction
    rng = np.random.default_rng(33)
    M, N, K = 3, 4, 64
    Xq, Xs = oracle.mxfp4_quantize(bf(rng.standard_normal((M, K))))
    Wq, Ws = oracle.mxfp4_quantize(bf(rng.standard_normal((N, K)) * 0.01))
    _, acc = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, want_acc=True)
    xd, wd = oracle.mxfp4_dequantize(Xq, Xs), oracle.mxfp4_dequantize(Wq, Ws)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xd[m], wd[n]))
            assert Fraction(float(acc[m, n])) == exact


def _fp4_grid_operands(rng, rows, K):
    """bf16 rows whose values lie on the FP4 grid with block exponent 0: every 32-element block
    holds a 4 or a 6, so its max is in [4, 8) and its scale is 2^0; the decoded values are then
    the values themselves (the lossless round trip is pinned above)."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    v = grid[rng.integers(0, 8, (rows, K))] * rng.choice([-1.0, 1.0], (rows, K))
    v[:, ::32] = rng.choice([-6.0, -4.0, 4.0, 6.0], (rows, K // 32))
    return v


def _bf16_rne_torch(x):
    """fp32 -> bf16 bit patterns through torch's own cast (round half to even), independent of
    the oracle's conversion."""
    torch = pytest.importorskip("torch")
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_mx_bias_epilogue_closed_form():
    # y = fp32(acc) + bias (one fp32 addition), then bf16: on grid operands acc is an exact
    # multiple of 1/4 computed here in integers, so the output is fixed by the closed form.
    # Dropping the bias, adding it after the bf16 rounding, or taking the wrong row's bias fails.
    rng = np.random.default_rng(36)
    M, N, K = 5, 48, 128
    xv, wv = _fp4_grid_operands(rng, M, K), _fp4_grid_operands(rng, N, K)
    Xq, Xs = oracle.mxfp4_quantize(bf(xv))
    Wq, Ws = oracle.mxfp4_quantize(bf(wv))
    assert np.all(Xs == 127) and np.all(Ws == 127)
    acc4 = (xv * 2).astype(np.int64) @ (wv * 2).astype(np.int64).T   # 4 acc, exact integers
    acc = acc4.astype(np.float64) / 4.0
    bias = bf(rng.standard_normal(N) * 40.0 + 0.3)
    Y, got_acc = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias, want_acc=True, epi="bias")
    assert np.array_equal(got_acc, acc)
    want = _bf16_rne_torch(acc.astype(np.float32) + f32(bias)[None, :])
    assert np.array_equal(Y, want)
    assert not np.array_equal(Y, _bf16_rne_torch(acc.astype(np.float32)))          # bias dropped
    assert not np.array_equal(Y, _bf16_rne_torch(acc.astype(np.float32) + f32(bias)[::-1][None, :]))
    # no bias: y = fp32(acc)
    Y0 = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, None, epi="bias")
    assert np.array_equal(Y0, _bf16_rne_torch(acc.astype(np.float32)))
    # selected rows are the same rows of the full result
    rows = np.array([4, 0, 2])
    assert np.array_equal(oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias, rows, epi="bias"), Y[rows])


def test_mx_silu_gate_epilogue_closed_form():
    # W rows [gate (0..F-1); up (F..2F-1)], g = fp32(acc_g) + b_g, u = fp32(acc_u) + b_u,
    # Y = bf16(silu(g) * u): within 1 bf16 ulp of the fp64 closed form on exact accumulators.
    # Gate and up are drawn with different scales, so swapping them, pairing gate f with up
    # row f + 1, or giving both halves the gate's bias moves some output by more than 1 ulp.
    from scipy.special import expit
    rng = np.random.default_rng(37)
    M, F, K = 6, 40, 96
    xv = _fp4_grid_operands(rng, M, K)
    wg, wu = _fp4_grid_operands(rng, F, K) * 0.125, _fp4_grid_operands(rng, F, K)
    Xq, Xs = oracle.mxfp4_quantize(bf(xv))
    Wq, Ws = oracle.mxfp4_quantize(bf(np.concatenate([wg, wu])))
    ag = (xv * 2).astype(np.int64) @ (wg * 16).astype(np.int64).T / 32.0   # exact
    au = (xv * 2).astype(np.int64) @ (wu * 2).astype(np.int64).T / 4.0
    bias = bf(np.concatenate([rng.standard_normal(F) * 0.5, rng.standard_normal(F) * 3.0 + 1.0]))
    bg, bu = f32(bias)[:F].astype(np.float64), f32(bias)[F:].astype(np.float64)
    Y, acc = oracle.mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias, want_acc=True, epi="silu_gate")
    assert Y.shape == (M, F)
    assert np.array_equal(acc[:, :F], ag) and np.array_equal(acc[:, F:], au)
    g = ag.astype(np.float32).astype(np.float64) + bg[None, :]
    u = au.astype(np.float32).astype(np.float64) + bu[None, :]
    want = g * expit(g) * u
    assert ulp_dist_bf16(Y, _bf16_rne_torch(want)).max() <= 1
    assert np.abs(g).max() > 4 and np.abs(u - g).max() > 4       # the two roles are far apart
    for wrong in (u * expit(u) * g,                               # gate and up swapped
                  g * expit(g) * np.roll(u, 1, axis=1),           # up row of the next gate
                  g * expit(g) * (u - bu + bg)):                  # the gate's bias on both halves
        assert ulp_dist_bf16(Y, _bf16_rne_torch(wrong)).max() > 1
    # zero gate gives zero; zero up gives zero
    Yz = oracle.mxfp4_gemm_rows(np.zeros_like(Xq), np.full_like(Xs, 0), Wq, Ws, None, epi="silu_gate")
    assert np.all(f32(Yz) == 0)


def test_bf16_gemm_within_fp64_bound():
    rng = np.random.default_rng(14)
    M, N, K = 9, 13, 512
    H = bf(rng.standard_normal((M, K)))
    Wd = bf(0.01 * rng.standard_normal((N, K)))
    bias = bf(0.01 * rng.standard_normal(N))
    Z, Zf = oracle.bf16_gemm_rows(H, Wd, bias, want_f32=True)
    ref = f32(H).astype(np.float64) @ f32(Wd).astype(np.float64).T + f32(bias).astype(np.float64)
    assert np.all(np.abs(Zf - ref) <= np.abs(ref) * 2.0 ** -24 + 1e-30)
    assert ulp_dist_bf16(Z, bf(ref.astype(np.float32))).max() <= 1
    rows = np.array([8, 0, 3])
    assert np.array_equal(oracle.bf16_gemm_rows(H, Wd, bias, rows), Z[rows])


# ----------------------------------------------------------------------------- page facts
def test_workload_shapes_match_page_facts():
    f = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    w = W.WORKLOADS
    hidden = f["hidden_width"]["value"]
    assert w["dit_attn_proj_4608x4608x4608"]["K"] == hidden == w["dit_attn_proj_4608x4608x4608"]["N"]
    assert w["dit_attn_proj_4608x4608x4608"]["M"] == f["packed_rows_1024"]["value"] \
        == f["text_rows_main_profile"]["value"] + f["image_rows_1024"]["value"]
    tc = w["text_cond_proj_512x4608x53248"]
    assert (tc["M"], tc["K"], tc["N"]) == (f["text_rows_main_profile"]["value"], f["qwen_feature_width"]["value"],
                                           hidden)
    assert [1, tc["padded_M"], tc["K"]] == f["conditioning_tensor_shape"]["value"]
    assert w["qk_proj_headnorm_6037x4608x4608"]["M"] == f["packed_rows_long_prompt"]["value"] \
        == f["packed_rows_long_prompt"]["prompt_tokens"] + f["image_rows_1024"]["value"]
    qk = w["qk_proj_headnorm_16896x4608x4608"]
    assert qk["M"] == f["predicted_zero_row_savings_gib"]["image_rows"][2] + f["text_rows_main_profile"]["value"]
    assert qk["head_dim"] == f["head_dim"]["value"] and qk["N"] % qk["head_dim"] == 0
    # byte counts printed on the page follow from these shapes
    c = f["cached_text_projection_mib"]
    assert math.prod(c["shape"]) * c["dtype_bytes"] / 2 ** 20 == c["value"]
    z = f["predicted_zero_row_savings_gib"]
    for rows, gib in zip(z["image_rows"], z["value"]):
        assert rows * tc["K"] * z["dtype_bytes"] * z["branches"] / 2 ** 30 == gib
    fc = f["fp32_construction_gib"]
    assert abs(sum(fc["rows"]) * fc["width"] * fc["dtype_bytes"] / 2 ** 30 - fc["value"]) < 5e-4
    assert W.BASE_SEED == f["seed"]["value"]


def test_generator_is_deterministic_and_prefix_stable():
    a = W.make_workload("tiny_w8a8_64x128x256")
    b = W.make_workload("tiny_w8a8_64x128x256")
    for k in ("X", "W", "bias"):
        assert np.array_equal(a[k], b[k])
    full = W.make_linear(70, 8, 256, seed=99, x_kind="pct1")
    pre = W.make_linear(30, 8, 256, seed=99, x_kind="pct1")
    assert np.array_equal(full["X"][:30], pre["X"])
    pad = W.make_linear(70, 8, 256, seed=99, x_kind="pct1", zero_rows_after=30)
    assert np.array_equal(pad["X"][:30], pre["X"]) and not pad["X"][30:].any()
    # outlier channels: 4 channels x20 in the tiny case
    fac = W.outlier_factors(256, 1000, "four20")
    assert sorted(np.unique(fac).tolist()) == [1.0, 20.0] and (fac == 20).sum() == 4


# ---------------------------------------------------------------- weight-only block formats
def test_f16_conversion_matches_numpy_and_saturates():
    """Round half to even with subnormals, checked against numpy's half conversion; from 65520
    up (where IEEE rounds to infinity) the reading saturates to 65504."""
    rng = np.random.default_rng(40)
    e = rng.integers(-30, 16, 4000)
    x = (rng.uniform(1, 2, 4000) * np.ldexp(1.0, e) * rng.choice([-1, 1], 4000)).astype(np.float32)
    # exact midpoints between neighbouring halves, normal and subnormal
    h = rng.integers(1, 0x7BFE, 500).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    x = np.concatenate([x, mid, np.float32([0.0, -0.0, 65504, 65519.99, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26])])
    got = oracle.f32_to_f16(x)
    assert np.array_equal(got, x.astype(np.float16).view(np.uint16))
    sat = oracle.f32_to_f16(np.float32([65520, -70000, 3e38]))
    assert list(sat) == [0x7BFF, 0xFBFF, 0x7BFF]


def test_f16_decode_every_finite_pattern():
    h = np.arange(0, 0x10000, dtype=np.uint16)
    h = h[(h & 0x7C00) != 0x7C00][::7]
    assert np.array_equal(oracle.f16_to_f64(h), h.view(np.float16).astype(np.float64))


def _wo_codes(Q, bits):
    """Signed codes [N, K] of weight-only blocks (test-side decoding of the documented layout)."""
    if bits == 8:
        return Q.astype(np.int64)
    q = np.empty((Q.shape[0], Q.shape[1] * 2), np.int64)
    q[:, 0::2] = (Q & 15).astype(np.int64) - 8
    q[:, 1::2] = (Q >> 4).astype(np.int64) - 8
    return q


@pytest.mark.parametrize("bits", [4, 8])
def test_wo_scale_rule_and_special_blocks(bits):
    qmax = 127 if bits == 8 else 7
    K = 32 * 6
    w = np.zeros((1, K), np.float32)
    rng = np.random.default_rng(41)
    # block 0: on the grid of d = 2^-7, with +-qmax present: exact codes
    g = rng.integers(-qmax, qmax + 1, 32)
    g[5] = -qmax
    w[0, :32] = g * 2.0 ** -7
    # block 1: all zero; block 2: amax / qmax underflows the half format (scale 0, codes 0)
    w[0, 64:96] = 1e-9 * rng.standard_normal(32)
    # block 3: amax / qmax is a half subnormal
    w[0, 96:128] = 3e-6 * rng.standard_normal(32)
    # block 4: amax / qmax above the half range: scale saturates, codes clamp
    w[0, 128:160] = 1e7 * rng.standard_normal(32)
    # block 5: one nonzero element
    w[0, 170] = -0.3
    Wb = bf(w)
    Q, D = oracle.wo_quantize(Wb, bits)
    q, d = _wo_codes(Q, bits), oracle.f16_to_f64(D)
    wv = f32(Wb).astype(np.float64)
    assert d[0, 0] == 2.0 ** -7 and np.array_equal(q[0, :32], g)
    assert d[0, 1] == 0 and np.all(q[0, 32:64] == 0)
    assert d[0, 2] == 0 and np.all(q[0, 64:96] == 0)
    assert 0 < d[0, 3] < 2.0 ** -14
    assert D[0, 4] == 0x7BFF and np.abs(q[0, 128:160]).max() == qmax
    # past the representable range every code saturates to +-qmax
    big = np.abs(wv[0, 128:160]) >= (qmax + 0.5) * 65504
    assert big.sum() >= 8 and np.array_equal(q[0, 128:160][big], qmax * np.sign(wv[0, 128:160][big]).astype(np.int64))
    assert q[0, 170] == -qmax and np.count_nonzero(q[0, 160:192]) == 1
    amax = np.abs(wv.reshape(6, 32)).max(axis=1)
    want = oracle.f32_to_f16((amax.astype(np.float32) / np.float32(qmax)).astype(np.float32))
    assert np.array_equal(D[0], want)


@pytest.mark.parametrize("bits", [4, 8])
def test_wo_codes_are_nearest_by_brute_force(bits):
    """Each code is the nearest grid point q * d (ties to even q) among all codes, away from
    exact-tie neighbourhoods where the fp32 division decides."""
    qmax = 127 if bits == 8 else 7
    rng = np.random.default_rng(42 + bits)
    Wb = bf(rng.standard_normal((16, 256)) * np.ldexp(1.0, rng.integers(-12, 2, (16, 1))))
    Q, D = oracle.wo_quantize(Wb, bits)
    q, d = _wo_codes(Q, bits), np.repeat(oracle.f16_to_f64(D), 32, axis=1)
    w = f32(Wb).astype(np.float64)
    grid = np.arange(-qmax, qmax + 1)
    dist = np.abs(w[..., None] - grid * d[..., None])
    best = dist.min(axis=-1, keepdims=True)
    cand = np.where(dist <= best * (1 + 1e-12), grid, 10 ** 6)
    even = np.where(cand % 2 == 0, cand, 10 ** 6).min(axis=-1)
    nearest = np.where((dist <= best * (1 + 1e-12)).sum(-1) > 1, even, grid[dist.argmin(-1)])
    t = w / d
    safe = np.abs(np.abs(t - np.floor(t)) - 0.5) > 1e-5
    assert np.array_equal(q[safe], nearest[safe])
    assert safe.mean() > 0.99


@pytest.mark.parametrize("bits", [4, 8])
def test_wo_exact_ties_round_to_even(bits):
    """Weights exactly halfway between grid points (d = 2^-6) take the even code."""
    qmax = 127 if bits == 8 else 7
    t = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, -5.5] * 4)
    t[0] = qmax                                   # sets d = 2^-6
    Q, D = oracle.wo_quantize(bf(t * 2.0 ** -6)[None, :], bits)
    assert oracle.f16_to_f64(D)[0, 0] == 2.0 ** -6
    want = np.array([0, 2, 2, 0, -2, -2, 4, -6] * 4)
    want[0] = qmax
    assert np.array_equal(_wo_codes(Q, bits)[0], want)


def test_wo_nibble_order_and_int8_layout():
    K = 64
    codes = (np.arange(K) % 15) - 7          # -7 .. 7
    w = bf(codes * 2.0 ** -4)                # block max 7 * 2^-4: d = 2^-4 for 4 bits
    Q4, D4 = oracle.wo_quantize(w[None, :], 4)
    assert list(D4[0]) == [0x2C00, 0x2C00]   # half 2^-4
    assert Q4[0, 0] == ((codes[0] + 8) | ((codes[1] + 8) << 4)) and Q4[0, 20] == ((codes[40] + 8) | ((codes[41] + 8) << 4))
    w8 = bf(((np.arange(K) * 37) % 255 - 127) * 2.0 ** -9)
    Q8, D8 = oracle.wo_quantize(w8[None, :], 8)
    assert Q8.dtype == np.int8 and np.array_equal(Q8[0].astype(np.int64), (np.arange(K) * 37) % 255 - 127)
    assert list(oracle.wo_dequantize(Q8, D8, 8)[0]) == list(w8)


@pytest.mark.parametrize("bits", [4, 8])
def test_wo_error_bound_and_dequant_rounding(bits):
    qmax = 127 if bits == 8 else 7
    rng = np.random.default_rng(44 + bits)
    Wb = bf(0.02 * rng.standard_normal((32, 512)))
    Q, D = oracle.wo_quantize(Wb, bits)
    w = f32(Wb).astype(np.float64)
    d = np.repeat(oracle.f16_to_f64(D), 32, axis=1)
    q = _wo_codes(Q, bits)
    amax = np.repeat(np.abs(w).reshape(32, 16, 32).max(axis=2), 32, axis=1)
    # half a grid step, or the clamp excess when the rounded scale fell below amax / qmax
    assert np.all(np.abs(w - q * d) <= np.maximum(d / 2, amax - qmax * d) * (1 + 1e-12))
    Wd = oracle.wo_dequantize(Q, D, bits)
    exact = q * d
    assert np.array_equal(Wd, bf(exact.astype(np.float32)))            # one rounding of the exact product
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)


@pytest.mark.parametrize("bits", [4, 8])
def test_wo_linear_exact_against_integer_matmul(bits):
    """On power-of-two scales the GEMM is an integer matmul times 2^-k: pins the operand
    layout (rows of W are output columns) and the bias."""
    qmax = 127 if bits == 8 else 7
    rng = np.random.default_rng(46 + bits)
    M, N, K = 5, 7, 128
    qi = rng.integers(-qmax, qmax + 1, (N, K))
    qi[:, ::32] = qmax                        # every block holds +qmax: d = 2^-6 exactly
    Q, D = oracle.wo_quantize(bf(qi * 2.0 ** -6), bits)
    assert np.array_equal(_wo_codes(Q, bits), qi)
    xi = rng.integers(-3, 4, (M, K))
    X = bf(xi * 0.5)
    bias = bf(rng.integers(-8, 9, N) * 0.25)
    Z, Zf = oracle.wo_linear_rows(X, Q, D, bits, bias, want_f32=True)
    want = (xi @ qi.T) * 2.0 ** -7 + f32(bias).astype(np.float64)
    assert np.array_equal(Zf.astype(np.float64), want)
    assert np.array_equal(Z, bf(want.astype(np.float32)))
    rows = np.array([4, 1])
    assert np.array_equal(oracle.wo_linear_rows(X, Q, D, bits, bias, rows), Z[rows])


# ---------------------------------------------------------------- attention
def _attn_inputs(S, H, ld, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    mk = lambda: bf(rng.standard_normal((S, ld)) * scale)
    return mk(), mk(), mk()


@pytest.mark.parametrize("h", [0, 2])
def test_attention_matches_library_softmax(h):
    """Against scipy's softmax on the same fp64 inputs; heads are column blocks of 256 inside ld."""
    from scipy.special import softmax
    S, H, ld = 96, 3, 3 * 256 + 8
    Q, K, V = _attn_inputs(S, H, ld, 50 + h, 1.5)
    rows = np.array([0, 5, 95, 40])
    O, A = oracle.attention_rows(Q, K, V, h, rows, want_f64=True)
    c = slice(256 * h, 256 * h + 256)
    q, k, v = (f32(T)[:, c].astype(np.float64) for T in (Q, K, V))
    ref = softmax(q[rows] @ k.T / 16.0, axis=1) @ v
    assert np.allclose(A, ref, rtol=1e-12, atol=1e-14)
    assert np.array_equal(O, bf(ref.astype(np.float32)))


def test_attention_uniform_scores_give_the_mean_of_v():
    """Zero queries score every key alike: the output is the plain mean of V, exact here."""
    S, ld = 64, 256
    rng = np.random.default_rng(52)
    Q = np.zeros((S, ld), np.uint16)
    K = bf(rng.standard_normal((S, ld)))
    vi = rng.integers(-8, 9, (S, ld))
    V = bf(vi * 0.25)
    O = oracle.attention_rows(Q, K, V, 0, np.array([0, 63]))
    want = bf((vi.sum(axis=0) * 0.25 / S).astype(np.float32))
    assert np.array_equal(O[0], want) and np.array_equal(O[1], want)


def test_attention_dominant_key_selects_its_value_row():
    """A key far ahead of the others (score gap 60) takes all the weight: the output is its V row."""
    S, ld = 48, 256
    rng = np.random.default_rng(53)
    Q = np.zeros((S, ld), np.float32)
    K = np.zeros((S, ld), np.float32)
    Q[:, 0] = 1.0
    K[:, 0] = rng.uniform(-1, 1, S)
    K[17, 0] = 960.0                      # score 60 above the rest
    V = bf(rng.standard_normal((S, ld)))
    O = oracle.attention_rows(bf(Q), bf(K), V, 0, np.array([3, 30]))
    assert np.array_equal(O[0], V[17]) and np.array_equal(O[1], V[17])


def test_attention_large_scores_stay_finite():
    """Scores around 4096 overflow exp unless the true row max is subtracted; with it the result
    is finite and equals the run with all scores shifted down by the same amount."""
    S, ld = 32, 256
    rng = np.random.default_rng(54)
    Q = np.zeros((S, ld), np.float32)
    K = np.zeros((S, ld), np.float32)
    Q[:, 0] = 64.0
    Q[:, 1] = 1.0
    K[:, 0] = 1024.0                      # scores 4096 + K[:, 1] / 16 ...
    K[:, 1] = rng.integers(-16, 17, S)
    K[0, 0] = 0.0                         # ... except key 0, 4096 below them (first is not the max)
    V = bf(rng.standard_normal((S, ld)))
    _, A = oracle.attention_rows(bf(Q), bf(K), V, 0, np.array([0]), want_f64=True)
    K2 = K.copy()
    K2[:, 0] = 0.0
    K2[0, 0] = -1024.0
    _, A2 = oracle.attention_rows(bf(Q), bf(K2), V, 0, np.array([0]), want_f64=True)
    assert np.all(np.isfinite(A)) and np.allclose(A, A2, rtol=1e-12, atol=1e-15)


def test_attention_key_permutation_and_other_heads():
    """Permuting keys with their values leaves the output (within fp64 rounding); the other
    heads' columns are never read."""
    S, ld = 80, 512
    Q, K, V = _attn_inputs(S, 2, ld, 55)
    perm = np.random.default_rng(56).permutation(S)
    _, A = oracle.attention_rows(Q, K, V, 1, np.array([7]), want_f64=True)
    _, Ap = oracle.attention_rows(Q, K[perm], V[perm], 1, np.array([7]), want_f64=True)
    assert np.allclose(A, Ap, rtol=1e-13, atol=1e-15)
    Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
    for T in (Q2, K2, V2):
        T[:, :256] = 0x7FC0              # NaN in head 0
    _, A2 = oracle.attention_rows(Q2, K2, V2, 1, np.array([7]), want_f64=True)
    assert np.array_equal(A, A2)
