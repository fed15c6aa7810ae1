"""Per-workload parity report (run by hand on a GPU machine; not collected by pytest).

For every workload of ``qdt_workloads.WORKLOADS`` it runs the whole path on the GPU, checks the
integer stages bit for bit against the oracle, and prints one JSON line with:

- the bf16 output's ulp histogram against the oracle on sampled rows (all rows of the tiny
  workload), and the bf16 down-projection's worst error as a fraction of its bound;
- the oracle's time on those rows and its extrapolation to the whole workload, with the host
  threads it used.

Usage:  python tests/config_report.py [--rows N] > report.jsonl
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import qdt_workloads as W  # noqa: E402
from qdt_testutil import bits_equal, sample_rows, to_dev, to_host, ulp_bf16  # noqa: E402


def histogram(u):
    vals, counts = np.unique(u, return_counts=True)
    return {str(int(v)): int(c) for v, c in zip(vals, counts)}


def run(name, nrows, qdt, torch, **kw):
    d = W.make_workload(name, **kw)
    M, N, K, epi = d["M"], d["N"], d["K"], d["epi"]
    t0 = time.perf_counter()
    s_r = oracle.channel_absmax(d["X"])
    Wq_r, sw_r, inv_r, _ = oracle.smooth_prepare(d["W"], s_r)
    Xq_r, sx_r = oracle.quantize_per_token(d["X"], inv_r)
    t_prep = time.perf_counter() - t0
    X, Wt = to_dev(d["X"]), to_dev(d["W"])
    s = qdt.channel_absmax(X)
    Wq, sw, inv, _ = qdt.smooth_prepare(Wt, s)
    Xq, sx = qdt.quantize_per_token(X, inv)
    gamma = to_dev(d["gamma"]) if d.get("gamma") is not None else None
    bias = to_dev(d["bias"]) if d.get("bias") is not None else None
    Y = qdt.w8a8_linear(Xq, sx, Wq, sw, bias, epi, gamma=gamma, eps=d.get("eps", 1e-6))
    torch.cuda.synchronize()
    exact = {k: bool(bits_equal(to_host(g), r)) for k, g, r in
             (("s", s, s_r), ("Wq", Wq, Wq_r), ("w_scale", sw, sw_r), ("Xq", Xq, Xq_r), ("x_scale", sx, sx_r))}
    rows = np.arange(M, dtype=np.int64) if M <= nrows else sample_rows(M, nrows, 7)
    t0 = time.perf_counter()
    Y_ref, acc_r = oracle.linear_rows(Xq_r, sx_r, Wq_r, sw_r, d.get("bias"), rows, epi, d.get("gamma"), 256,
                                      d.get("eps", 1e-6), want_acc=True)
    t_rows = time.perf_counter() - t0
    Yh = to_host(Y)
    out = dict(workload=name + ("_padded" if kw.get("padded") else ""), M=M, N=N, K=K, epilogue=epi,
               integer_stages_bit_exact=exact, rows_compared=int(rows.size),
               ulp_histogram=histogram(ulp_bf16(Yh[rows], Y_ref)),
               oracle_threads=oracle.threads(), oracle_prepare_and_quantize_s=round(t_prep, 3),
               oracle_linear_s_on_rows=round(t_rows, 3),
               oracle_linear_s_whole_workload_est=round(t_rows * M / rows.size, 1))
    if epi == "bias":
        Ya = qdt.w8a8_linear(Xq, sx, Wq, sw, None, "acc_i32")
        torch.cuda.synchronize()
        out["acc_i32_bit_exact_on_rows"] = bool(np.array_equal(to_host(Ya)[rows], acc_r))
    if "W_down" in d:
        rr = rows[:16]
        Hf = W.bf16_bits_to_f32(Yh[rr]).astype(np.float64)
        Wf = W.bf16_bits_to_f32(d["W_down"]).astype(np.float64)
        Z = to_host(qdt.bf16_linear(Y, to_dev(d["W_down"])))[rr]
        zref = Hf @ Wf.T
        Kd = Yh.shape[1]
        gam = Kd * 2.0 ** -24 / (1 - Kd * 2.0 ** -24)
        bound = gam * (np.abs(Hf) @ np.abs(Wf).T) + 2.0 ** (np.floor(np.log2(np.maximum(np.abs(zref), 2.0 ** -126))) - 7)
        err = np.abs(W.bf16_bits_to_f32(Z).astype(np.float64) - zref)
        out["bf16_down_proj"] = dict(rows_compared=int(rr.size), worst_err_over_bound=float((err / bound).max()),
                                     ulp_histogram=histogram(ulp_bf16(Z, oracle.bf16_gemm_rows(Yh, d["W_down"], rows=rr))))
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--rows", type=int, default=96, help="sampled rows per workload")
    a = ap.parse_args()
    import torch
    import quantized_diffusion_transformer_amd as qdt
    for name in W.WORKLOADS:
        print(f"[case] {name}", file=sys.stderr, flush=True)
        run(name, a.rows, qdt, torch)
        if name.startswith("text_cond_proj"):
            print(f"[case] {name} padded", file=sys.stderr, flush=True)
            run(name, a.rows, qdt, torch, padded=True)


if __name__ == "__main__":
    main()
