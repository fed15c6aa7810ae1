"""Parity of the attention after the QK-norm projection (qdt_attention) against the oracle.

Exact cases compare bit for bit:
- uniform scores, where the output is the mean of V with power-of-two key counts;
- a dominant key, where the output is its V row, both below the kernel's rerun threshold and far
  above it, which forces the exact-max rerun.

General inputs are gated by a first-order error bound of the kernel's arithmetic:
- bf16 probabilities: relative 2^-9;
- the exponential and its argument: 2^-21;
- fp32 scores: gamma_256 * sum_d |q_d k_d| scaled by ln 2 / 16 through the exponent;
- fp32 sums of S terms for the numerator and the denominator.
The resulting relative error multiplies sum_j p_j |v_j| / sum_j p_j, and the final bf16 rounding
adds one ulp of the result.
"""
import numpy as np
import pytest

import oracle
import qdt_workloads as W
from qdt_testutil import bits_equal, to_dev, to_host, ulp_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
qdt = pytest.importorskip("quantized_diffusion_transformer_amd")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def bf(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


def f64(b):
    return W.bf16_bits_to_f32(b).astype(np.float64)


def run(Q, K, V, H, ld_pad=0):
    """qdt_attention on bf16 bit arrays [S, 256 H] (stored with ld = 256 H + ld_pad, NaN padding)."""
    S = Q.shape[0]
    if ld_pad:
        pads = []
        for T in (Q, K, V):
            P = np.full((S, 256 * H + ld_pad), 0x7FC0, np.uint16)
            P[:, :256 * H] = T
            pads.append(to_dev(P)[:, :256 * H])
        return to_host(qdt.attention(*pads, H))
    return to_host(qdt.attention(to_dev(Q), to_dev(K), to_dev(V), H))


def within_bound(O, Q, K, V, h, rows):
    """Checks O's rows against the oracle within the first-order bound; returns the fraction of
    outputs equal to the oracle's correctly rounded result."""
    c = slice(256 * h, 256 * h + 256)
    q, k, v = f64(Q)[rows][:, c], f64(K)[:, c], f64(V)[:, c]
    S = k.shape[0]
    s = q @ k.T / 16.0
    p = np.exp(s - s.max(axis=1, keepdims=True))
    l = p.sum(axis=1, keepdims=True)
    A = (p @ np.abs(v)) / l
    E = np.abs(q) @ np.abs(k).T                                   # sum_d |q_d k_d|
    g256 = 256 * 2.0 ** -24 / (1 - 256 * 2.0 ** -24)
    gS = S * 2.0 ** -24 / (1 - S * 2.0 ** -24)
    score = np.log(2.0) * (1.4426950408889634 / 16.0) * g256 * E.max(axis=1, keepdims=True) * 1.01
    rel = 2.0 ** -9 + 2.0 ** -21 + 2 * score + 2 * gS
    O_ref, acc = oracle.attention_rows(Q, K, V, h, rows, want_f64=True)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(acc), 2.0 ** -126))) - 7)
    got = f64(O[rows][:, c])
    err = np.abs(got - acc)
    bound = rel * A * 1.25 + ulp
    assert np.all(err <= bound), f"worst error / bound {np.max(err / bound):.3f}"
    return float(np.mean(O[rows][:, c] == O_ref))


@pytest.mark.parametrize("S,H", [(64, 1), (128, 2), (4096, 1), (16384, 1)])
def test_attention_uniform_scores_exact(S, H):
    """Zero queries: every probability is exactly 1, the output is the mean of V (exact in fp32 for
    power-of-two key counts), bit for bit.  Up to 8192 tokens the kernel reads V transposed in LDS,
    past it from a V^T written first (16384): both paths."""
    announce(f"attention uniform S={S} H={H}")
    rng = np.random.default_rng(900 + S)
    Q = np.zeros((S, 256 * H), np.uint16)
    K = bf(rng.standard_normal((S, 256 * H)))
    V = bf(rng.integers(-8, 9, (S, 256 * H)) * 0.25)
    O = run(Q, K, V, H)
    rows = np.array([0, S // 2, S - 1])
    for h in range(H):
        assert bits_equal(O[rows][:, 256 * h:256 * h + 256], oracle.attention_rows(Q, K, V, h, rows))


@pytest.mark.parametrize("gap,key,exact", [(400.0, 5, True), (400.0, 70, False), (4000.0, 70, True)])
def test_attention_dominant_key_exact(gap, key, exact):
    """One key scores `gap` (raw q.k) above all others: the output is its V row.
    - Key 5 is the first key tile's max, the reference, so its probability is exactly 1.
    - Key 70 lies in the third tile.  With gap 400 its probability is 2^35.4 against the first tile's
      reference; it enters the second product as bf16 (relative 2^-9), while the row sum keeps
      fp32, so the output is within 1 bf16 ulp of the row.
    - With gap 4000 (360 in log2 units, past the limit of 64) the workgroup is recomputed with the
      exact max, and the probability is 1 again."""
    announce(f"attention dominant key {key} gap {gap}")
    S, H = 100, 1
    rng = np.random.default_rng(910)
    Q = np.zeros((S, 256), np.float32)
    K = np.zeros((S, 256), np.float32)
    Q[:, 0] = 1.0
    Q[:, 1] = rng.uniform(-1, 1, S)
    K[:, 0] = rng.integers(-4, 5, S)
    K[:, 1] = rng.integers(-4, 5, S)
    K[key, 0] = gap
    V = bf(rng.standard_normal((S, 256)))
    O = run(bf(Q), bf(K), V, H)
    want = np.broadcast_to(V[key], O.shape)
    if exact:
        assert np.array_equal(O, want)
    else:
        assert ulp_bf16(O, want).max() <= 1


@pytest.mark.parametrize("S", [8192, 8200])
def test_attention_dominant_key_rerun_exact_at_the_path_boundary(S):
    """The exact-max rerun on both sides of the 8192-token switch between V read transposed in LDS
    and the V^T pass: key S - 3 (in the partial last key tile of 8200) scores 4000 above the rest,
    past the 64 log2-unit limit, so every workgroup is recomputed with the exact max and its output
    is that key's V row bit for bit."""
    announce(f"attention dominant key rerun S={S}")
    rng = np.random.default_rng(920 + S)
    key = S - 3
    Q = np.zeros((S, 256), np.float32)
    K = np.zeros((S, 256), np.float32)
    Q[:, 0] = 1.0
    K[:, 0] = rng.integers(-4, 5, S)
    K[key, 0] = 4000.0
    V = bf(rng.standard_normal((S, 256)))
    O = run(bf(Q), bf(K), V, 1)
    assert np.array_equal(O, np.broadcast_to(V[key], O.shape))


@pytest.mark.parametrize("S,H,pad", [(300, 2, 24), (1, 1, 0), (33, 3, 8)])
def test_attention_within_bound(S, H, pad):
    """QK-norm-like inputs (unit RMS per head, a per-dimension gain), ragged S against the 32-key
    tiles and the 256-query blocks, rows stored with NaN padding past 256 H."""
    announce(f"attention bound S={S} H={H} pad={pad}")
    rng = np.random.default_rng(920 + S)
    gain = np.exp(rng.normal(0, 0.3, 256 * H))
    Q = bf(rng.standard_normal((S, 256 * H)) * gain)
    K = bf(rng.standard_normal((S, 256 * H)) * gain)
    V = bf(rng.standard_normal((S, 256 * H)))
    O = run(Q, K, V, H, pad)
    rows = np.arange(S)
    for h in range(H):
        within_bound(O, Q, K, V, h, rows)


def test_attention_query_rows_are_independent():
    """Permuting the query rows permutes the output rows, bit for bit."""
    announce("attention query permutation")
    S, H = 600, 1
    rng = np.random.default_rng(930)
    Q = bf(rng.standard_normal((S, 256)))
    K = bf(rng.standard_normal((S, 256)))
    V = bf(rng.standard_normal((S, 256)))
    O = to_host(qdt.attention(to_dev(Q), to_dev(K), to_dev(V), H))
    perm = rng.permutation(S)
    O2 = to_host(qdt.attention(to_dev(Q[perm]), to_dev(K), to_dev(V), H))
    assert bits_equal(O2, O[perm])


def test_attention_full_size_sampled_rows():
    """The 2048^2 joint sequence: 16896 tokens, 18 heads of 256, sampled query rows of two heads."""
    d = W.make_attention(16896, 18)
    announce("attention 16896 x 18 heads")
    O = to_host(qdt.attention(to_dev(d["Q"]), to_dev(d["K"]), to_dev(d["V"]), 18))
    rows = np.array([0, 1, 255, 256, 8000, 16639, 16640, 16895])
    for h in (0, 17):
        exact = within_bound(O, d["Q"], d["K"], d["V"], h, rows)
        print(f"head {h}: {exact:.3f} of the sampled outputs equal the correctly rounded result", flush=True)


def test_attention_ragged_full_heads_sampled_rows():
    """6037 tokens (21 keys past the last full 32-key tile, 149 queries past the last full 256-query
    block), all 18 heads, sampled rows of three heads including the last query row."""
    d = W.make_attention(6037, 18, seed=W.BASE_SEED + 5)
    announce("attention 6037 x 18 heads")
    O = to_host(qdt.attention(to_dev(d["Q"]), to_dev(d["K"]), to_dev(d["V"]), 18))
    rows = np.array([0, 255, 256, 5887, 5888, 6000, 6036])
    for h in (0, 9, 17):
        within_bound(O, d["Q"], d["K"], d["V"], h, rows)


# Shapes whose last round of workgroups is split into key ranges (qdt.h, qdt_attention): 2048 tokens
# x 40 heads has 320 (query block, head) tiles; the 64 past one round of 256 (heads 32-39) run as 4
# key ranges of 512 keys each, merged afterwards.  4608 x 18 (the attention after the 4608-token
# projection) splits its last 68 tiles (head 14 from query 1024 on, heads 15-17) into 3 ranges.


def test_attention_split_uniform_scores_exact():
    """Zero queries with key-range pieces: every piece's probabilities are exactly 1 against the same
    reference, so the merged output is the exact mean of V, bit for bit, in whole and split heads."""
    S, H = 2048, 40
    announce(f"attention split uniform S={S} H={H}")
    rng = np.random.default_rng(940)
    Q = np.zeros((S, 256 * H), np.uint16)
    K = bf(rng.standard_normal((S, 256 * H)))
    V = bf(rng.integers(-8, 9, (S, 256 * H)) * 0.25)
    O = run(Q, K, V, H)
    rows = np.array([0, 1000, S - 1])
    for h in (0, 31, 32, 39):
        assert bits_equal(O[rows][:, 256 * h:256 * h + 256], oracle.attention_rows(Q, K, V, h, rows)), f"head {h}"


def test_attention_split_dominant_key_rerun_exact():
    """A key 4000 raw points above the rest, inside the second key range of the split heads and past
    that range's first tile: that piece is recomputed with its exact max, the other pieces' weights
    2^(c_i - M) underflow to zero, and every output row is the key's V row, bit for bit."""
    S, H, key = 2048, 40, 1000
    announce(f"attention split dominant key S={S} H={H}")
    rng = np.random.default_rng(950)
    Q = np.zeros((S, 256 * H), np.float32)
    K = np.zeros((S, 256 * H), np.float32)
    for h in range(H):
        Q[:, 256 * h] = 1.0
        K[:, 256 * h] = rng.integers(-4, 5, S)
        K[key, 256 * h] = 4000.0
    V = bf(rng.standard_normal((S, 256 * H)))
    O = run(bf(Q), bf(K), V, H)
    for h in (0, 39):
        c = slice(256 * h, 256 * h + 256)
        assert np.array_equal(O[:, c], np.broadcast_to(V[key, c], (S, 256))), f"head {h}"


def test_attention_split_full_size_sampled_rows():
    """4608 tokens x 18 heads, the split layout: sampled rows of a whole head (0), a head that is
    whole up to query 1023 and split after (14) and a split head (17), within the same bound."""
    d = W.make_attention(4608, 18, seed=W.BASE_SEED + 1)
    announce("attention 4608 x 18 heads (split last round)")
    O = to_host(qdt.attention(to_dev(d["Q"]), to_dev(d["K"]), to_dev(d["V"]), 18))
    rows = np.array([0, 255, 1023, 1024, 2500, 4607])
    for h in (0, 14, 17):
        exact = within_bound(O, d["Q"], d["K"], d["V"], h, rows)
        print(f"head {h}: {exact:.3f} of the sampled outputs equal the correctly rounded result", flush=True)
