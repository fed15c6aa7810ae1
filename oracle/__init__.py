"""ctypes front end of the CPU oracle (``qdt_oracle.c``).

TEST INFRASTRUCTURE: imported only by the test suite, the smoke check and the
benchmark's CPU-baseline leg.  It shares nothing with the HIP path.  Arrays are
numpy; bf16 tensors travel as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "qdt_oracle.c")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-pthread", "-Wall"]

EPI_BIAS, EPI_SILU_GATE, EPI_HEAD_RMSNORM = 0, 1, 2
_EPI = {"bias": EPI_BIAS, "silu_gate": EPI_SILU_GATE, "head_rmsnorm": EPI_HEAD_RMSNORM}


def compile_oracle() -> str:
    cmd = ["gcc", *CFLAGS, SRC_PATH, "-o", LIB_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            compile_oracle()
        L = C.CDLL(LIB_PATH)
        P, I64, F, I = C.c_void_p, C.c_int64, C.c_float, C.c_int
        sig = {
            "oracle_version": ([], I),
            "oracle_set_threads": ([I], None),
            "oracle_threads": ([], I),
            "oracle_bf16_to_f32": ([C.c_uint16], F),
            "oracle_f32_to_bf16": ([F], C.c_uint16),
            "oracle_f32_to_bf16_array": ([P, P, I64], None),
            "oracle_channel_absmax": ([P, I64, I64, I64, P, I], None),
            "oracle_smooth_lambda": ([P, P, I64, F, P, P], None),
            "oracle_quantize_rows": ([P, P, I64, I64, I64, P, P], None),
            "oracle_smooth_prepare": ([P, P, I64, I64, F, P, P, P, P], None),
            "oracle_gemm_i32": ([P, P, I64, I64, I64, P], None),
            "oracle_gemm_i64": ([P, P, I64, I64, I64, P], None),
            "oracle_epilogue": ([P, I64, I64, P, P, P, I, P, I64, F, P, I64], None),
            "oracle_linear_rows": ([P, P, P, P, P, P, I64, I64, I64, I, P, I64, F, P, I64, P], None),
            "oracle_bf16_gemm_rows": ([P, P, P, P, I64, I64, I64, P, P], None),
            "oracle_adaln_modulate": ([P, I64, I64, I64, P, P, F, P], None),
            "oracle_fp4_value": ([I], C.c_double),
            "oracle_mxfp4_quantize_rows": ([P, P, I64, I64, I64, P, P], None),
            "oracle_mxfp4_gemm_rows": ([P, P, P, P, P, P, I64, I64, I64, I, P, F, P, P], None),
            "oracle_f32_to_f16": ([F], C.c_uint16),
            "oracle_f16_to_f64": ([C.c_uint16], C.c_double),
            "oracle_wo_quantize": ([P, I64, I64, I64, I, P, P], None),
            "oracle_wo_dequantize": ([P, P, I64, I64, I, P], None),
            "oracle_attention_rows": ([P, P, P, I64, I64, I64, P, I64, P, P], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def threads() -> int:
    return int(lib().oracle_threads())


def f32_to_bf16(x) -> np.ndarray:
    x = _c(np.atleast_1d(x), np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16_array(_p(x), _p(out), x.size)
    return out


def channel_absmax(X: np.ndarray, s: np.ndarray | None = None) -> np.ndarray:
    X = _c(X, np.uint16)
    M, K = X.shape
    acc = s is not None
    s = np.zeros(K, np.float32) if s is None else _c(s, np.float32).copy()
    lib().oracle_channel_absmax(_p(X), M, K, K, _p(s), int(acc))
    return s


def smooth_lambda(s, w, alpha: float = 0.5):
    s, w = _c(s, np.float32), _c(w, np.float32)
    lam = np.empty_like(s)
    inv = np.empty_like(s)
    lib().oracle_smooth_lambda(_p(s), _p(w), s.size, alpha, _p(lam), _p(inv))
    return lam, inv


def quantize_rows(X: np.ndarray, colmul: np.ndarray | None = None):
    X = _c(X, np.uint16)
    M, K = X.shape
    q = np.empty((M, K), np.int8)
    sc = np.empty(M, np.float32)
    lib().oracle_quantize_rows(_p(X), _p(_c(colmul, np.float32)), M, K, K, _p(q), _p(sc))
    return q, sc


def quantize_per_token(X: np.ndarray, inv_lambda: np.ndarray | None):
    return quantize_rows(X, inv_lambda)


def smooth_prepare(W: np.ndarray, s: np.ndarray | None, alpha: float = 0.5):
    """Returns (Wq int8 [N,K], sw f32 [N], inv_lambda f32 [K], lambda f32 [K])."""
    W = _c(W, np.uint16)
    N, K = W.shape
    Wq = np.empty((N, K), np.int8)
    sw = np.empty(N, np.float32)
    inv = np.empty(K, np.float32)
    lam = np.empty(K, np.float32)
    lib().oracle_smooth_prepare(_p(W), _p(_c(s, np.float32)), N, K, alpha, _p(Wq), _p(sw), _p(inv), _p(lam))
    return Wq, sw, inv, lam


def gemm_i32(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    A, B = _c(A, np.int8), _c(B, np.int8)
    M, K = A.shape
    N = B.shape[0]
    out = np.empty((M, N), np.int32)
    lib().oracle_gemm_i32(_p(A), _p(B), M, N, K, _p(out))
    return out


def gemm_i64(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    A, B = _c(A, np.int8), _c(B, np.int8)
    M, K = A.shape
    N = B.shape[0]
    out = np.empty((M, N), np.int64)
    lib().oracle_gemm_i64(_p(A), _p(B), M, N, K, _p(out))
    return out


def _n_out(N: int, epi: int) -> int:
    return N // 2 if epi == EPI_SILU_GATE else N


def epilogue(acc, sx, sw, bias=None, epi="bias", gamma=None, head_dim=256, eps=1e-6) -> np.ndarray:
    e = _EPI[epi] if isinstance(epi, str) else int(epi)
    acc = _c(acc, np.int32)
    M, N = acc.shape
    no = _n_out(N, e)
    Y = np.empty((M, no), np.uint16)
    lib().oracle_epilogue(_p(acc), M, N, _p(_c(sx, np.float32)), _p(_c(sw, np.float32)), _p(_c(bias, np.uint16)),
                          e, _p(_c(gamma, np.uint16)), head_dim, eps, _p(Y), no)
    return Y


def linear_rows(Xq, sx, Wq, sw, bias, rows, epi="bias", gamma=None, head_dim=256, eps=1e-6, want_acc=False):
    """GEMM + epilogue for the given rows; returns Y rows (and int32 acc rows when want_acc)."""
    e = _EPI[epi] if isinstance(epi, str) else int(epi)
    Xq, Wq = _c(Xq, np.int8), _c(Wq, np.int8)
    rows = _c(rows, np.int64)
    N, K = Wq.shape
    no = _n_out(N, e)
    Y = np.empty((rows.size, no), np.uint16)
    acc = np.empty((rows.size, N), np.int32) if want_acc else None
    lib().oracle_linear_rows(_p(Xq), _p(_c(sx, np.float32)), _p(Wq), _p(_c(sw, np.float32)),
                             _p(_c(bias, np.uint16)), _p(rows), rows.size, N, K, e, _p(_c(gamma, np.uint16)),
                             head_dim, eps, _p(Y), no, _p(acc))
    return (Y, acc) if want_acc else Y


def linear(X, W, bias=None, s=None, alpha=0.5, epi="bias", gamma=None, head_dim=256, eps=1e-6):
    """The whole path on the CPU: prepare, quantize, GEMM, epilogue.  Returns a dict of stages."""
    s = channel_absmax(X) if s is None else s
    Wq, sw, inv, lam = smooth_prepare(W, s, alpha)
    Xq, sx = quantize_per_token(X, inv)
    acc = gemm_i32(Xq, Wq)
    Y = epilogue(acc, sx, sw, bias, epi, gamma, head_dim, eps)
    return dict(s=s, Wq=Wq, sw=sw, inv_lambda=inv, lam=lam, Xq=Xq, sx=sx, acc=acc, Y=Y)


def bf16_gemm_rows(H, W, bias=None, rows=None, want_f32=False):
    H, W = _c(H, np.uint16), _c(W, np.uint16)
    M, K = H.shape
    N = W.shape[0]
    r = None if rows is None else _c(rows, np.int64)
    nr = M if r is None else r.size
    Z = np.empty((nr, N), np.uint16)
    Zf = np.empty((nr, N), np.float32) if want_f32 else None
    lib().oracle_bf16_gemm_rows(_p(H), _p(W), _p(_c(bias, np.uint16)), _p(r), nr, N, K, _p(Z), _p(Zf))
    return (Z, Zf) if want_f32 else Z


def adaln_modulate(X, shift=None, scale=None, eps: float = 1e-6) -> np.ndarray:
    """bf16 [M,K] = bf16(LayerNorm(X) * (1 + scale) + shift), the input of the next linear."""
    X = _c(X, np.uint16)
    M, K = X.shape
    H = np.empty((M, K), np.uint16)
    lib().oracle_adaln_modulate(_p(X), M, K, K, _p(_c(shift, np.uint16)), _p(_c(scale, np.uint16)), eps, _p(H))
    return H


def adaln_quantize(X, shift, scale, inv_lambda, eps: float = 1e-6):
    """The fused producer's three outputs on the CPU: (Xq, x_scale, H)."""
    H = adaln_modulate(X, shift, scale, eps)
    Xq, sx = quantize_rows(H, inv_lambda)
    return Xq, sx, H


def fp4_value(code: int) -> float:
    return float(lib().oracle_fp4_value(int(code)))


def mxfp4_quantize(X, colmul=None):
    """Block-scaled FP4 of bf16 X [M,K] (times colmul): (codes uint8 [M,K/2], exponents uint8 [M,K/32])."""
    X = _c(X, np.uint16)
    M, K = X.shape
    Q = np.zeros((M, K // 2), np.uint8)
    S = np.empty((M, K // 32), np.uint8)
    lib().oracle_mxfp4_quantize_rows(_p(X), _p(_c(colmul, np.float32)), M, K, K, _p(Q), _p(S))
    return Q, S


def mxfp4_dequantize(Q, S) -> np.ndarray:
    """fp64 values of block-scaled FP4 rows (for tests)."""
    Q, S = np.asarray(Q, np.uint8), np.asarray(S, np.uint8)
    codes = np.empty((Q.shape[0], Q.shape[1] * 2), np.int64)
    codes[:, 0::2] = Q & 15
    codes[:, 1::2] = Q >> 4
    table = np.array([fp4_value(c) for c in range(16)])
    return table[codes] * np.ldexp(1.0, np.repeat(S.astype(np.int64) - 127, 32, axis=1))


def mxfp4_gemm_rows(Xq, Xs, Wq, Ws, bias=None, rows=None, want_acc=False, epi="bias", gamma=None, eps=1e-6):
    """fp64 accumulators of the decoded product and the bf16 output of epilogue ``epi`` ("bias":
    bf16((float)acc + bias); "silu_gate": W rows [gate; up], bf16(silu(g) * u); "head_rmsnorm":
    per 256-column head with gamma) for the given rows."""
    e = _EPI[epi]
    Xq, Xs, Wq, Ws = (_c(a, np.uint8) for a in (Xq, Xs, Wq, Ws))
    N, K = Wq.shape[0], Wq.shape[1] * 2
    r = None if rows is None else _c(rows, np.int64)
    nr = Xq.shape[0] if r is None else r.size
    Y = np.empty((nr, _n_out(N, e)), np.uint16)
    acc = np.empty((nr, N), np.float64) if want_acc else None
    lib().oracle_mxfp4_gemm_rows(_p(Xq), _p(Xs), _p(Wq), _p(Ws), _p(_c(bias, np.uint16)), _p(r), nr, N, K, e,
                                 _p(_c(gamma, np.uint16)), eps, _p(acc), _p(Y))
    return (Y, acc) if want_acc else Y


def f32_to_f16(x) -> np.ndarray:
    """IEEE half bits of fp32 values: round half to even, saturating at 65504."""
    a = np.asarray(x, np.float32).ravel()
    L = lib()
    return np.array([L.oracle_f32_to_f16(float(v)) for v in a], np.uint16).reshape(np.shape(x))


def f16_to_f64(h) -> np.ndarray:
    a = np.asarray(h, np.uint16).ravel()
    L = lib()
    return np.array([L.oracle_f16_to_f64(int(v)) for v in a], np.float64).reshape(np.shape(h))


def wo_quantize(W, bits: int = 4):
    """Weight-only blocks of W [N, K] bf16 (K % 32 == 0): codes (int8 [N, K] for 8 bits, nibbles
    uint8 [N, K/2] for 4 bits) and half-precision scale bits uint16 [N, K/32]."""
    assert bits in (4, 8)
    W = np.asarray(W, np.uint16)
    N, K = W.shape
    ldw = W.strides[0] // 2
    Q = np.zeros((N, K if bits == 8 else K // 2), np.int8 if bits == 8 else np.uint8)
    D = np.empty((N, K // 32), np.uint16)
    if W.strides[1] != 2:
        W = np.ascontiguousarray(W)
        ldw = K
    lib().oracle_wo_quantize(_p(W), N, K, ldw, bits, _p(Q), _p(D))
    return Q, D


def wo_dequantize(Q, D, bits: int) -> np.ndarray:
    """bf16 [N, K] = bf16(q * d) of weight-only blocks."""
    Q = _c(Q, np.int8 if bits == 8 else np.uint8)
    D = _c(D, np.uint16)
    N = Q.shape[0]
    K = D.shape[1] * 32
    Wd = np.empty((N, K), np.uint16)
    lib().oracle_wo_dequantize(_p(Q), _p(D), N, K, bits, _p(Wd))
    return Wd


def wo_linear_rows(X, Q, D, bits: int, bias=None, rows=None, want_f32=False):
    """The weight-only linear: the bf16 GEMM of X with the dequantized weights (plus bias)."""
    return bf16_gemm_rows(X, wo_dequantize(Q, D, bits), bias, rows, want_f32)


def attention_rows(Q, K, V, h: int, rows=None, want_f64=False):
    """Head h of softmax(Q K^T / 16) V for the listed query rows: bf16 [n, 256] (and fp64 values).
    Q, K, V: bf16 bits [S, ld] with head h in columns 256 h .. 256 h + 255."""
    Q, K, V = _c(Q, np.uint16), _c(K, np.uint16), _c(V, np.uint16)
    S, ld = Q.shape
    r = None if rows is None else _c(rows, np.int64)
    n = S if r is None else r.size
    O = np.empty((n, 256), np.uint16)
    A = np.empty((n, 256), np.float64) if want_f64 else None
    lib().oracle_attention_rows(_p(Q), _p(K), _p(V), S, ld, h, _p(r), n, _p(O), _p(A))
    return (O, A) if want_f64 else O
