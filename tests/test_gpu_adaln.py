"""Parity of the producer-fused quantizer (qdt_adaln_quantize) against the oracle.

The adaLN output h is gated at 1 bf16 ulp (the mean and variance are fp32 sums on the GPU and
fp64 sums in the oracle), and must be exact on almost every element.  The int8 codes and the
per-token scales are gated bit for bit against the oracle's quantizer applied to the GPU's own h,
so both sides take each rounding decision on the same values.
"""
import numpy as np
import pytest

import oracle
import qdt_workloads as W
from qdt_testutil import bits_equal, sample_rows, to_dev, to_host, ulp_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
qdt = pytest.importorskip("quantized_diffusion_transformer_amd")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def consumer_inv_lambda(d, H_ref):
    """Smoothing vector of the linear that consumes h: from h's column max-abs and W's."""
    s = oracle.channel_absmax(H_ref)
    w = oracle.channel_absmax(d["W"])
    _, inv = oracle.smooth_lambda(s, w)
    return inv


def run_and_check(d, use_shift=True, use_scale=True, use_inv=True, eps=1e-6, ldx=None, rows=None):
    M, K = d["M"], d["K"]
    sh = d["shift"] if use_shift else None
    sc = d["scale"] if use_scale else None
    H_ref = oracle.adaln_modulate(d["X"], sh, sc, eps)
    inv = consumer_inv_lambda(d, H_ref) if use_inv else None
    Xh = d["X"]
    if ldx is not None:
        Xh = np.zeros((M, ldx), np.uint16)
        Xh[:, :K] = d["X"]
        Xh[:, K:] = 0x7FC0  # NaN in the padding columns: must never be read
    Xd = to_dev(Xh)[:, :K] if ldx is not None else to_dev(Xh)
    args = (Xd, None if sh is None else to_dev(sh), None if sc is None else to_dev(sc),
            None if inv is None else to_dev(inv))
    Xq, sx, H = qdt.adaln_quantize(*args, eps=eps, want_h=True)
    Xq2, sx2 = qdt.adaln_quantize(*args, eps=eps)
    torch.cuda.synchronize()
    Hg, Xqg, sxg = to_host(H), to_host(Xq), to_host(sx)
    u = ulp_bf16(Hg, H_ref)
    assert u.max() <= 1, f"h: max ulp {u.max()}"
    assert np.mean(u == 0) > 0.999, f"h exact on only {np.mean(u == 0):.5f} of the elements"
    q_ref, s_ref = oracle.quantize_rows(Hg, inv)
    assert bits_equal(Xqg, q_ref), f"Xq: {np.sum(Xqg != q_ref)} codes differ"
    assert bits_equal(sxg, s_ref), f"x_scale: {np.sum(sxg != s_ref)} scales differ"
    # writing h or not changes nothing else; the adaLN alone writes the same h
    assert bits_equal(to_host(Xq2), Xqg) and bits_equal(to_host(sx2), sxg)
    assert bits_equal(to_host(qdt.adaln_modulate(args[0], args[1], args[2], eps=eps)), Hg)
    return Hg, Xqg, sxg, inv


# (the last four: rows whose last chunks cover only some lanes, with 6, 9, 12 and 16 chunks per lane;
# such lanes load the row's last chunk again and skip it)
@pytest.mark.parametrize("M,K", [(1, 64), (37, 256), (129, 512), (67, 4608), (40, 8192), (300, 1088),
                                 (61, 3008), (50, 4160), (33, 5696), (45, 7744)])
def test_adaln_quantize_parity(M, K):
    announce(f"adaln_quantize M={M} K={K}")
    run_and_check(W.make_adaln(M, K, seed=3000 + K))


@pytest.mark.parametrize("flags", [(False, False, False), (True, False, True), (False, True, False),
                                   (True, True, False)])
def test_adaln_optional_vectors(flags):
    announce(f"adaln_quantize optional shift/scale/inv_lambda {flags}")
    run_and_check(W.make_adaln(70, 1024, seed=3100), *flags)


def test_adaln_row_stride_and_eps():
    announce("adaln_quantize ldx > K, eps 1e-2")
    d = W.make_adaln(33, 2048, seed=3200)
    d["X"][5] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(d["X"][5]) * np.float32(1e-2))  # variance ~ eps
    run_and_check(d, ldx=2048 + 72, eps=1e-2)
    # a row whose last chunk covers only some lanes, in a wider buffer
    run_and_check(W.make_adaln(29, 4160, seed=3201), ldx=4160 + 200)


def test_adaln_constant_and_zero_rows_give_shift():
    announce("adaln_quantize constant rows")
    d = W.make_adaln(6, 512, seed=3300)
    vals = [0.0, 1.0, -3.25, 1e4, 7e-30, -0.5]
    d["X"] = np.repeat(W.f32_to_bf16_bits(np.array(vals, np.float32))[:, None], 512, axis=1)
    Hg, Xqg, sxg, inv = run_and_check(d)
    assert np.array_equal(Hg, np.broadcast_to(d["shift"], Hg.shape))


def test_adaln_full_size_4608_then_linear():
    """The DiT hidden width at 4608 tokens, every row compared; then the consumer linear on the
    fused Xq matches the oracle's linear on sampled rows bit for bit (BIAS epilogue)."""
    announce("adaln_quantize 4608x4608 + w8a8_linear")
    d = W.make_adaln(4608, 4608)
    Hg, Xqg, sxg, inv = run_and_check(d)
    s = oracle.channel_absmax(Hg)
    Wq_r, sw_r, inv_r, _ = oracle.smooth_prepare(d["W"], s)
    Wq, sw, inv_g, _ = qdt.smooth_prepare(to_dev(d["W"]), to_dev(s))
    Xq, sx = qdt.adaln_quantize(to_dev(d["X"]), to_dev(d["shift"]), to_dev(d["scale"]), inv_g)
    bias = W.vector(4608, 3400, 3, 0.01)
    Y = to_host(qdt.w8a8_linear(Xq, sx, Wq, sw, to_dev(bias), "bias"))
    q_ref, s_ref = oracle.quantize_rows(Hg, inv_r)
    assert bits_equal(to_host(Xq), q_ref) and bits_equal(to_host(sx), s_ref)
    rows = sample_rows(4608, 24, 9)
    Y_ref = oracle.linear_rows(q_ref, s_ref, Wq_r, sw_r, bias, rows, "bias")
    assert bits_equal(Y[rows], Y_ref)
