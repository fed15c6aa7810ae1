"""Per-workload report: the bf16 output's ulp histogram against the oracle, and the accuracy of
the quantized linear against unquantized arithmetic, with and without smoothing.

For every workload of ``qdt_workloads.WORKLOADS`` (and the zero-padded text projection) the whole
path runs on the GPU, and one JSON line is printed (``[report] {...}``; also appended to the file
named by the environment variable QDT_REPORT_JSONL when it is set) with:

- ``ulp_histogram``: the bf16 output against the oracle on sampled rows (all rows of the tiny
  workload); the integer stages are checked bit for bit;
- ``accuracy``: relative Frobenius error and largest absolute error of the W8A8 output against
  the same linear in fp64 on the bf16 inputs (X Wᵀ + b, then the workload's epilogue: gated SiLU,
  or the head RMSNorm with gamma), once with SmoothQuant (alpha 0.5, calibrated on the workload's
  X) and once without smoothing (lambda = 1).  This is the synthetic counterpart of the
  activation-quantization ablation in the results paragraph of "Quantizing a Dual-Branch
  Flow-Matching Diffusion Transformer for Consumer GPUs": naive per-token INT8 suffers from the
  outlier channels, smoothing recovers most of the error.  The magnitudes are information only;
  the one property asserted is the direction (smoothing lowers the error on these inputs, all of
  which carry outlier channels);
- the oracle's time on the sampled rows, and its extrapolation to the whole workload, with the
  host threads it used.
"""
import json
import os
import time

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

ROWS = 32
CASES = [(n, False) for n in W.WORKLOADS] + [("text_cond_proj_512x4608x53248", True)]


def histogram(u):
    vals, counts = np.unique(u, return_counts=True)
    return {str(int(v)): int(c) for v, c in zip(vals, counts)}


def fp64_reference(d, rows):
    """The workload's linear in fp64 on the bf16 inputs, for the given rows: y = X Wᵀ + b, then the
    epilogue (SiLU(g) u on the [gate; up] halves, or RMSNorm per 256-wide head times gamma)."""
    from scipy.special import expit
    Xf = W.bf16_bits_to_f32(d["X"][rows]).astype(np.float64)
    Wf = W.bf16_bits_to_f32(d["W"]).astype(np.float64)
    y = Xf @ Wf.T
    if d.get("bias") is not None:
        y += W.bf16_bits_to_f32(d["bias"]).astype(np.float64)[None, :]
    if d["epi"] == "silu_gate":
        F = y.shape[1] // 2
        return y[:, :F] * expit(y[:, :F]) * y[:, F:]
    if d["epi"] == "head_rmsnorm":
        g = W.bf16_bits_to_f32(d["gamma"]).astype(np.float64)
        h = y.reshape(len(rows), -1, 256)
        return (h / np.sqrt((h ** 2).mean(axis=2, keepdims=True) + d["eps"]) * g).reshape(len(rows), -1)
    return y


def gpu_linear(d, smooth):
    X, Wt = to_dev(d["X"]), to_dev(d["W"])
    s = qdt.channel_absmax(X) if smooth else None
    Wq, sw, inv, _ = qdt.smooth_prepare(Wt, s)
    Xq, sx = qdt.quantize_per_token(X, inv if smooth else None)
    gamma = to_dev(d["gamma"]) if d.get("gamma") is not None else None
    bias = to_dev(d["bias"]) if d.get("bias") is not None else None
    Y = qdt.w8a8_linear(Xq, sx, Wq, sw, bias, d["epi"], gamma=gamma, eps=d.get("eps", 1e-6))
    torch.cuda.synchronize()
    return dict(s=s, Wq=Wq, sw=sw, Xq=Xq, sx=sx, Y=to_host(Y))


@pytest.mark.parametrize("name,padded", CASES, ids=[n + ("_padded" if p else "") for n, p in CASES])
def test_workload_report(name, padded):
    print(f"[case] report {name}{' padded' if padded else ''}", flush=True)
    d = W.make_workload(name, padded=padded)
    M, N, K, epi = d["M"], d["N"], d["K"], d["epi"]
    t0 = time.perf_counter()
    s_r = oracle.channel_absmax(d["X"])
    Wq_r, sw_r, inv_r, _ = oracle.smooth_prepare(d["W"], s_r)
    Xq_r, sx_r = oracle.quantize_per_token(d["X"], inv_r)
    t_prep = time.perf_counter() - t0
    g = gpu_linear(d, smooth=True)
    for k, r in (("s", s_r), ("Wq", Wq_r), ("sw", sw_r), ("Xq", Xq_r), ("sx", sx_r)):
        assert bits_equal(to_host(g[k]), r), f"{k} differs from the oracle"
    real = 512 if padded else M  # padded: the text rows carry the information; the zero rows give the bias
    rows = np.arange(real, dtype=np.int64) if real <= 2 * ROWS else sample_rows(real, ROWS, 7)
    t0 = time.perf_counter()
    Y_ref = oracle.linear_rows(Xq_r, sx_r, Wq_r, sw_r, d.get("bias"), rows, epi, d.get("gamma"), 256,
                               d.get("eps", 1e-6))
    t_rows = time.perf_counter() - t0
    u = ulp_bf16(g["Y"][rows], Y_ref)
    assert u.max() <= (0 if epi == "bias" else 1)
    ref = fp64_reference(d, rows)
    acc = {}
    for label, Y in (("smoothquant_alpha_0.5", g["Y"]), ("no_smoothing", gpu_linear(d, smooth=False)["Y"])):
        e = W.bf16_bits_to_f32(Y[rows]).astype(np.float64) - ref
        acc[label] = {"rel_frobenius": float(np.linalg.norm(e) / np.linalg.norm(ref)),
                      "max_abs": float(np.abs(e).max())}
    out = dict(workload=name + ("_padded" if padded else ""), M=M, N=N, K=K, epilogue=epi,
               rows_compared=int(rows.size), ulp_histogram=histogram(u),
               accuracy_vs_fp64_unquantized=acc,
               oracle_threads=oracle.threads(), oracle_prepare_and_quantize_s=round(t_prep, 3),
               oracle_linear_s_on_rows=round(t_rows, 3),
               oracle_linear_s_whole_workload_est=round(t_rows * M / rows.size, 1))
    line = json.dumps(out)
    print(f"[report] {line}", flush=True)
    path = os.environ.get("QDT_REPORT_JSONL")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")
    # the direction of the ablation on these outlier-carrying inputs (information otherwise)
    assert acc["smoothquant_alpha_0.5"]["rel_frobenius"] < acc["no_smoothing"]["rel_frobenius"]
