"""The hot path captured in a HIP graph (torch.cuda.graph) replays bit-identically.

Every entry point enqueues only kernels on the caller's stream (no memsets, no allocation, no
host synchronization), so a step can be captured and replayed.  Each test captures the step
once, then replays it several times with unrelated eager work and synchronizations between the
replays, and compares every replay with the eager result bit for bit.
"""
import numpy as np
import pytest

import qdt_workloads as W
from qdt_testutil import bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
qdt = pytest.importorskip("quantized_diffusion_transformer_amd")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def replay_and_compare(step, outs, want, reps=4):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream before capturing
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    junk = torch.randn(1024, 1024, device="cuda")
    for r in range(reps):
        for o in outs:
            o.zero_()
        junk = junk @ junk.T / 1024.0  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert bits_equal(to_host(o), w), f"replay {r}: output differs from the eager result"


@pytest.mark.parametrize("M,N,K,split", [(64, 128, 256, None), (600, 1024, 4096, 4), (4608, 4608, 4608, None)])
def test_quantize_and_linear_in_a_graph(M, N, K, split):
    announce(f"graph: quantize + w8a8_linear M={M} N={N} K={K} split={split}")
    d = W.make_linear(M, N, K, seed=5000 + M, bias=True)
    X, Wt, b = to_dev(d["X"]), to_dev(d["W"]), to_dev(d["bias"])
    Wq, sw, inv, _ = qdt.smooth_prepare(Wt, qdt.channel_absmax(X))
    plan = qdt.linear_plan(M, N, K, "bias", split_k=split)
    ws = torch.empty(max(plan["workspace_bytes"], 16), dtype=torch.uint8, device="cuda")
    Xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        qdt.quantize_per_token(X, inv, Xq, sx)
        qdt.w8a8_linear(Xq, sx, Wq, sw, b, "bias", out=Y, workspace=ws, split_k=split)
    step()
    torch.cuda.synchronize()
    want = [to_host(Xq), to_host(sx), to_host(Y)]
    replay_and_compare(step, [Xq, sx, Y], want)


def test_adaln_producer_and_fp4_in_a_graph():
    announce("graph: adaln_quantize + mxfp4 path")
    d = W.make_adaln(512, 4608)
    X, sh, sc = to_dev(d["X"]), to_dev(d["shift"]), to_dev(d["scale"])
    inv = torch.rand(4608, device="cuda") + 0.5
    Xq = torch.empty((512, 4608), dtype=torch.int8, device="cuda")
    sx = torch.empty(512, dtype=torch.float32, device="cuda")
    Wq4, Ws4 = qdt.mxfp4_quantize(to_dev(d["W"][:1024]))
    Q4 = torch.empty((512, 2304), dtype=torch.uint8, device="cuda")
    S4 = torch.empty((18, 512, 8), dtype=torch.uint8, device="cuda")
    Y4 = torch.empty((512, 1024), dtype=torch.bfloat16, device="cuda")

    def step():
        qdt.adaln_quantize(X, sh, sc, inv, Xq=Xq, x_scale=sx)
        qdt.mxfp4_quantize(X, None, Q4, S4)
        qdt.mxfp4_linear(Q4, S4, Wq4, Ws4, None, out=Y4)
    step()
    torch.cuda.synchronize()
    want = [to_host(t) for t in (Xq, sx, Q4, S4, Y4)]
    replay_and_compare(step, [Xq, sx, Q4, S4, Y4], want)
