"""The allocation-free W8A8 linear (qdt_w8a8_linear_noalloc) against qdt_w8a8_linear with its own
workspace: bit-identical outputs on two calls in a row through the C ABI, the second smaller than
the first (the static scratch keeps the first call's partial sums, which the second must not see),
and the size limit reported on the host before any launch."""
import ctypes as C

import numpy as np
import pytest

import oracle
import qdt_workloads as W
from qdt_testutil import bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
qdt = pytest.importorskip("quantized_diffusion_transformer_amd")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def operands(M, N, K, seed, epi="bias"):
    d = W.make_linear(M, N, K, seed=seed, x_kind="pct1", epi=epi)
    X, Wt = to_dev(d["X"]), to_dev(d["W"])
    s = qdt.channel_absmax(X)
    Wq, sw, inv, _ = qdt.smooth_prepare(Wt, s)
    Xq, sx = qdt.quantize_per_token(X, inv)
    return d, Xq, sx, Wq, sw


def noalloc_call(Xq, sx, Wq, sw, b, epi, Y, params=None):
    """qdt_w8a8_linear_noalloc through the C ABI; returns the status."""
    M, K = Xq.shape
    N = Wq.shape[0]
    p = None if params is None else C.cast(C.byref(params), C.c_void_p)
    return qdt.qdt_w8a8_linear_noalloc(Xq.data_ptr(), sx.data_ptr(), Wq.data_ptr(), sw.data_ptr(),
                                       None if b is None else b.data_ptr(), M, N, K, qdt.EPILOGUES[epi], p,
                                       Y.data_ptr(), Y.stride(0), C.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("epi", ["bias", "head_rmsnorm", "silu_gate"])
def test_noalloc_matches_workspace_path_two_calls(epi):
    # call 1 splits K 4 ways over a larger output, call 2 13 ways over a smaller one: the second
    # call's partial sums overwrite part of what the first left in the scratch
    cases = [(300, 1024, 16384, 5), (64, 512, 53248, 6)]
    for M, N, K, seed in cases:
        announce(f"noalloc {epi} M={M} N={N} K={K}")
        plan = qdt.linear_plan(M, N, K, epi)
        assert plan["split_k"] > 1 and plan["workspace_bytes"] <= qdt.QDT_NOALLOC_SCRATCH_BYTES
        d, Xq, sx, Wq, sw = operands(M, N, K, seed, epi)
        b = to_dev(d["bias"])
        kw, params = {}, None
        if epi == "head_rmsnorm":
            g = to_dev(d["gamma"])
            kw = dict(gamma=g, eps=d["eps"])
            params = qdt.qdt_rmsnorm_params(g.data_ptr(), 256, d["eps"])
        ref = qdt.w8a8_linear(Xq, sx, Wq, sw, b, epi, **kw)
        nout = N // 2 if epi == "silu_gate" else N
        Y = torch.full((M, nout), 7, dtype=torch.bfloat16, device="cuda")
        assert noalloc_call(Xq, sx, Wq, sw, b, epi, Y, params) == qdt.QDT_OK
        torch.cuda.synchronize()
        assert bits_equal(to_host(Y), to_host(ref)), f"{epi} M={M}: outputs differ"
        if epi == "bias":  # and the oracle on a few rows
            rows = np.array([0, M // 2, M - 1], np.int64)
            s_r = oracle.channel_absmax(d["X"])
            Wq_r, sw_r, inv_r, _ = oracle.smooth_prepare(d["W"], s_r)
            Xq_r, sx_r = oracle.quantize_per_token(d["X"], inv_r)
            Y_r = oracle.linear_rows(Xq_r, sx_r, Wq_r, sw_r, d["bias"], rows, "bias")
            assert bits_equal(to_host(Y)[rows], Y_r)


def test_noalloc_unsplit_and_binding():
    announce("noalloc unsplit / binding")
    d, Xq, sx, Wq, sw = operands(600, 1152, 2048, 8)
    b = to_dev(d["bias"])
    assert qdt.linear_plan(600, 1152, 2048, "bias")["split_k"] == 1
    ref = qdt.w8a8_linear(Xq, sx, Wq, sw, b, "bias")
    Y = torch.empty_like(ref)
    qdt.w8a8_linear_noalloc(Xq, sx, Wq, sw, b, "bias", out=Y)
    torch.cuda.synchronize()
    assert bits_equal(to_host(Y), to_host(ref))


def test_noalloc_rejects_plans_beyond_the_scratch():
    # 512 rows x 11008 outputs of the 53248-deep projection split 3 ways need 67.6 MB of partial
    # sums: refused on the host with QDT_EWORKSPACE, nothing launched (no device memory is touched)
    M, N, K = 512, 11008, 53248
    plan = qdt.linear_plan(M, N, K, "bias")
    assert plan["workspace_bytes"] > qdt.QDT_NOALLOC_SCRATCH_BYTES
    Xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    Wq = torch.empty((N, K), dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    sw = torch.empty(N, dtype=torch.float32, device="cuda")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    st = qdt.qdt_w8a8_linear_noalloc(Xq.data_ptr(), sx.data_ptr(), Wq.data_ptr(), sw.data_ptr(), None, M, N, K,
                                     qdt.QDT_EPI_BIAS, None, Y.data_ptr(), N, None)
    assert st == qdt.QDT_EWORKSPACE
