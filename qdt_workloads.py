"""Seeded synthetic inputs for the W8A8 DiT linear.

This module only draws random tensors with the shapes, distributions and
structure of the DiT linears described in the pages; it holds none of the
method's arithmetic (no smoothing, no quantization, no GEMM).  Both the CPU
oracle (``oracle/``) and the HIP path take their inputs from here.

Shapes follow the pages:
  * hidden width 4608 and 4096 image + 512 text positions at 1024^2, 6037
    positions with a 1941-token prompt -- "Faster Ideogram 4 with Less Prompt
    Compute", section "Conditioning a Denoising Step";
  * the 53248-wide Qwen feature rows projected to 4608 with a bias, text rows
    first and 4096 all-zero image rows after them -- same page, sections
    "Conditioning a Denoising Step" and "Most of the Tensor Was Zero";
  * 256-dimensional attention heads -- "Serving sub-second Ideogram v4 without
    quality loss", paragraph on fused epilogues;
  * 16384 image positions at 2048^2 (the pages' zero-row savings at 512^2,
    1024^2 and 2048^2 scale as 1024, 4096 and 16384 rows).

Distributions (N(mu, sigma) with sigma the standard deviation) are the ones the
workload table names; where it leaves a choice open (which channels are
outliers, the factor law of the heavy tail, the FFN weight scales) the choice
made here is stated next to the code.

Random streams: numpy PCG64 seeded with SeedSequence([seed, tensor_id]); every
tensor is drawn in fp32 and rounded to bf16 with round-half-to-even.
"""
from __future__ import annotations

import numpy as np

# tensor ids for SeedSequence([seed, tensor_id])
_TID_X, _TID_W, _TID_BIAS, _TID_GAMMA, _TID_WDOWN, _TID_OUTCH, _TID_OUTF = 1, 2, 3, 4, 5, 6, 7
_TID_SHIFT, _TID_SCALE = 8, 9
_TID_Q, _TID_K, _TID_V, _TID_GQ, _TID_GK = 10, 11, 12, 13, 14

BASE_SEED = 1000  # the fixed generation seed of the INT8/GGUF quantization paper's setup


def rng_for(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id)])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (round half to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, sigma: float, mean: float = 0.0,
                 col_factor: np.ndarray | None = None, rows_per_chunk: int = 1024) -> np.ndarray:
    """N(mean, sigma) drawn in fp32 row-chunk by row-chunk, optional per-column factor, then bf16."""
    rows, cols = shape
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, rows_per_chunk):
        r1 = min(rows, r0 + rows_per_chunk)
        z = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if sigma != 1.0:
            z *= np.float32(sigma)
        if mean != 0.0:
            z += np.float32(mean)
        if col_factor is not None:
            z *= col_factor[None, :]
        out[r0:r1] = f32_to_bf16_bits(z)
    return out


def outlier_factors(K: int, seed: int, kind: str) -> np.ndarray:
    """Per-channel multipliers for the activation outlier channels.

    kind:
      "four20"  -- 4 channels scaled x20 (the tiny case);
      "pct1"    -- 1% of channels (round(0.01*K)) scaled by U[10, 50] each;
      "pareto"  -- 1% of channels scaled by a classical Pareto(x_min=10, shape 1.5)
                   factor clipped at 1000 (our reading of "heavy-tailed outliers");
      "none"    -- no outliers.
    Channels are a seeded choice without replacement.
    """
    f = np.ones(K, dtype=np.float32)
    if kind == "none":
        return f
    rc = rng_for(seed, _TID_OUTCH)
    rf = rng_for(seed, _TID_OUTF)
    if kind == "four20":
        n = min(4, K)
        ch = rc.choice(K, size=n, replace=False)
        f[ch] = 20.0
    elif kind == "pct1":
        n = max(1, int(round(0.01 * K)))
        ch = rc.choice(K, size=n, replace=False)
        f[ch] = rf.uniform(10.0, 50.0, size=n).astype(np.float32)
    elif kind == "pareto":
        n = max(1, int(round(0.01 * K)))
        ch = rc.choice(K, size=n, replace=False)
        fac = (rf.pareto(1.5, size=n) + 1.0) * 10.0
        f[ch] = np.minimum(fac, 1000.0).astype(np.float32)
    else:
        raise ValueError(f"unknown outlier kind {kind!r}")
    return f


def activations(M: int, K: int, seed: int, kind: str, zero_rows_after: int | None = None) -> np.ndarray:
    """X bf16 [M, K] ~ N(0, 1) with outlier channels.  Rows >= zero_rows_after are all zero."""
    f = outlier_factors(K, seed, kind)
    rows = M if zero_rows_after is None else min(M, zero_rows_after)
    x = np.zeros((M, K), dtype=np.uint16)
    if rows > 0:
        x[:rows] = _normal_bf16(rng_for(seed, _TID_X), (rows, K), 1.0, col_factor=f)
    return x


def weights(N: int, K: int, seed: int, sigma: float, tensor_id: int = _TID_W) -> np.ndarray:
    return _normal_bf16(rng_for(seed, tensor_id), (N, K), sigma)


def vector(n: int, seed: int, tensor_id: int, sigma: float, mean: float = 0.0) -> np.ndarray:
    return _normal_bf16(rng_for(seed, tensor_id), (1, n), sigma, mean=mean)[0]


# --------------------------------------------------------------------------------------
# The five workloads.  Names say what they are; "epi" is the fused op after the GEMM.
# --------------------------------------------------------------------------------------
WORKLOADS = {
    "tiny_w8a8_64x128x256": dict(M=64, N=128, K=256, seed=BASE_SEED + 0, x_kind="four20",
                                 w_sigma=0.02, bias=True, epi="bias"),
    "dit_attn_proj_4608x4608x4608": dict(M=4608, N=4608, K=4608, seed=BASE_SEED + 1, x_kind="pct1",
                                         w_sigma=0.015, bias=True, epi="bias"),
    # X is the attention-projection X (same seed); gate and up rows stacked as [gate; up].
    "dit_ffn_gate_up_4608x24576x4608": dict(M=4608, N=24576, K=4608, seed=BASE_SEED + 1, x_kind="pct1",
                                            w_seed=BASE_SEED + 2, w_sigma=0.015, bias=False, epi="silu_gate",
                                            down_K=12288, down_N=4608, down_sigma=0.01),
    "text_cond_proj_512x4608x53248": dict(M=512, N=4608, K=53248, seed=BASE_SEED + 3, x_kind="pareto",
                                          w_sigma=0.005, bias=True, epi="bias", padded_M=4608),
    "qk_proj_headnorm_16896x4608x4608": dict(M=16896, N=4608, K=4608, seed=BASE_SEED + 4, x_kind="pct1",
                                             w_sigma=0.015, bias=True, epi="head_rmsnorm",
                                             head_dim=256, eps=1e-6, gamma_sigma=0.1),
    "qk_proj_headnorm_6037x4608x4608": dict(M=6037, N=4608, K=4608, seed=BASE_SEED + 5, x_kind="pct1",
                                            w_sigma=0.015, bias=True, epi="head_rmsnorm",
                                            head_dim=256, eps=1e-6, gamma_sigma=0.1),
}

HEADLINE = "dit_attn_proj_4608x4608x4608"


def make_linear(M: int, N: int, K: int, seed: int, x_kind: str = "pct1", w_sigma: float = 0.015,
                bias: bool = True, epi: str = "bias", w_seed: int | None = None,
                zero_rows_after: int | None = None, head_dim: int = 256, eps: float = 1e-6,
                gamma_sigma: float = 0.1, **_ignored) -> dict:
    """Inputs of one W8A8 linear at any shape, with a workload's distributions.

    Returns bf16 bit patterns (uint16): X [M,K], W [N,K], bias [N] (or None),
    gamma [head_dim] for the head-norm epilogue.
    """
    ws = seed if w_seed is None else w_seed
    d = dict(M=M, N=N, K=K, seed=seed, epi=epi)
    d["X"] = activations(M, K, seed, x_kind, zero_rows_after=zero_rows_after)
    d["W"] = weights(N, K, ws, w_sigma)
    d["bias"] = vector(N, ws, _TID_BIAS, 0.01) if bias else None
    if epi == "head_rmsnorm":
        d["gamma"] = vector(head_dim, ws, _TID_GAMMA, gamma_sigma, mean=1.0)
        d["head_dim"] = head_dim
        d["eps"] = eps
    return d


def make_workload(name: str, M: int | None = None, padded: bool = False) -> dict:
    """Inputs of a named workload; ``M`` overrides the row count (rows stay the seeded prefix)."""
    cfg = dict(WORKLOADS[name])
    if padded:
        rows = cfg["M"]
        cfg["M"] = cfg["padded_M"]
        d = make_linear(zero_rows_after=rows, **cfg)
    else:
        if M is not None:
            cfg["M"] = M
        d = make_linear(**cfg)
    if "down_K" in cfg:
        d["W_down"] = weights(cfg["down_N"], cfg["down_K"], cfg.get("w_seed", cfg["seed"]),
                              cfg["down_sigma"], tensor_id=_TID_WDOWN)
    d["name"] = name
    return d


def make_adaln(M: int, K: int, seed: int = BASE_SEED + 1, x_kind: str = "pct1", shift_sigma: float = 0.25,
               scale_sigma: float = 0.5, w_sigma: float = 0.015) -> dict:
    """Inputs of the adaLN producer in front of a quantized linear: the residual stream X (the
    attention projection's recipe and seed by default), the run-time modulation vectors shift
    and scale [K] (a synthetic choice: the pages print no values), and a weight W [K, K] of the
    consumer linear whose column max-abs enters the smoothing vector."""
    return dict(M=M, K=K, seed=seed, X=activations(M, K, seed, x_kind),
                shift=vector(K, seed, _TID_SHIFT, shift_sigma), scale=vector(K, seed, _TID_SCALE, scale_sigma),
                W=weights(K, K, seed, w_sigma))


def make_attention(S: int, H: int, seed: int = BASE_SEED + 4) -> dict:
    """Inputs of the attention after the QK-norm projection: Q and K as that projection's head
    RMSNorm leaves them (unit mean square per head, times a per-dimension gain gamma ~ N(1, 0.1)
    shared by all heads: a synthetic choice, the pages print no weights), V ~ N(0, 1), all bf16
    [S, 256 H] token-major, head h in columns 256 h .. 256 h + 255."""
    gq = np.tile(1.0 + 0.1 * rng_for(seed, _TID_GQ).standard_normal(256, dtype=np.float32), H).astype(np.float32)
    gk = np.tile(1.0 + 0.1 * rng_for(seed, _TID_GK).standard_normal(256, dtype=np.float32), H).astype(np.float32)
    return dict(S=S, H=H, seed=seed,
                Q=_normal_bf16(rng_for(seed, _TID_Q), (S, 256 * H), 1.0, col_factor=gq),
                K=_normal_bf16(rng_for(seed, _TID_K), (S, 256 * H), 1.0, col_factor=gk),
                V=_normal_bf16(rng_for(seed, _TID_V), (S, 256 * H), 1.0))
