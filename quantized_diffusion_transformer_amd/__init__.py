"""Python binding of libqdt.so, the HIP (gfx950) W8A8 quantized linear of a flow-matching DiT.

Argument marshalling only: every step runs in the library's kernels.  torch supplies the
device memory and the current stream.  The ctypes entry points keep the C names
(``qdt_quantize_per_token`` ...); the torch-facing helpers drop the prefix
(``quantize_per_token`` ...), allocate outputs with torch and raise on any non-OK status.

Importing this module loads the library and fails loudly if it has not been built
(``python -c "import __graft_entry__ as g; g.build()"``).
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqdt.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libqdt.so not found at {LIB_PATH}: build the HIP library first "
                      "(quantized_diffusion_transformer_amd/_build.py)")

_lib = C.CDLL(LIB_PATH)

# ------------------------------------------------------------------------------- C types
QDT_OK, QDT_EINVAL, QDT_ESHAPE, QDT_EALIGN, QDT_EWORKSPACE, QDT_EALIAS, QDT_EHIP, QDT_EUNSUPPORTED = range(8)
QDT_EPI_BIAS, QDT_EPI_SILU_GATE, QDT_EPI_HEAD_RMSNORM, QDT_EPI_ACC_I32, QDT_EPI_ACC_F32 = range(5)
QDT_TILE_AUTO, QDT_TILE_256, QDT_TILE_288, QDT_TILE_288x256, QDT_TILE_224x256 = -1, 0, 1, 2, 3
QDT_MAX_K = 131072
QDT_MAX_ADALN_K = 8192

EPILOGUES = {"bias": QDT_EPI_BIAS, "silu_gate": QDT_EPI_SILU_GATE, "head_rmsnorm": QDT_EPI_HEAD_RMSNORM,
             "acc_i32": QDT_EPI_ACC_I32}


class qdt_rmsnorm_params(C.Structure):
    _fields_ = [("gamma", C.c_void_p), ("head_dim", C.c_int32), ("eps", C.c_float)]


class qdt_linear_plan(C.Structure):
    _fields_ = [("tile", C.c_int32), ("split_k", C.c_int32), ("tile_m", C.c_int32), ("tile_n", C.c_int32),
                ("tiles_m", C.c_int32), ("tiles_n", C.c_int32), ("k_tiles", C.c_int32), ("grid", C.c_int32),
                ("workspace_bytes", C.c_int64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_P, _I64, _F, _I, _SZ = C.c_void_p, C.c_int64, C.c_float, C.c_int, C.c_size_t
_SIGS = {
    "qdt_status_string": ([_I], C.c_char_p),
    "qdt_version": ([], C.c_char_p),
    "qdt_channel_absmax": ([_P, _I64, _I64, _I64, _P, _I, _P], _I),
    "qdt_smooth_prepare": ([_P, _P, _I64, _I64, _F, _P, _P, _P, _P, _P], _I),
    "qdt_quantize_per_token": ([_P, _P, _I64, _I64, _I64, _P, _P, _P], _I),
    "qdt_adaln_quantize": ([_P, _I64, _P, _P, _F, _P, _I64, _I64, _P, _P, _P, _P], _I),
    "qdt_mxfp4_quantize": ([_P, _P, _I64, _I64, _I64, _P, _P, _P], _I),
    "qdt_mxfp4_linear": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _I64, _P, _SZ, _P], _I),
    "qdt_mxfp4_linear_plan": ([_I64, _I64, _I64, _I, C.POINTER(qdt_linear_plan)], _I),
    "qdt_mxfp4_linear_plan_for": ([_I64, _I64, _I64, _I, C.c_int32, C.c_int32, C.POINTER(qdt_linear_plan)], _I),
    "qdt_mxfp4_linear_planned": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _I64, _P, _SZ,
                                  C.POINTER(qdt_linear_plan), _P], _I),
    "qdt_wo_quantize": ([_P, _I64, _I64, _I64, _I, _P, _P, _P], _I),
    "qdt_wo_linear": ([_P, _I64, _P, _P, _I, _P, _I64, _I64, _I64, _I, _P, _I64, _P, _SZ, _P], _I),
    "qdt_wo_linear_plan": ([_I64, _I64, _I64, C.POINTER(qdt_linear_plan)], _I),
    "qdt_attention": ([_P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _SZ, _P], _I),
    "qdt_attention_workspace_size": ([_I64, _I64, C.POINTER(_SZ)], _I),
    "qdt_w8a8_linear_plan": ([_I64, _I64, _I64, _I, C.POINTER(qdt_linear_plan)], _I),
    "qdt_w8a8_linear_plan_for": ([_I64, _I64, _I64, _I, C.c_int32, C.c_int32, C.POINTER(qdt_linear_plan)], _I),
    "qdt_w8a8_linear_workspace_size": ([_I64, _I64, _I64, _I, C.POINTER(_SZ)], _I),
    "qdt_w8a8_linear": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _I64, _P, _SZ, _P], _I),
    "qdt_w8a8_linear_planned": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _I64, _P, _SZ,
                                 C.POINTER(qdt_linear_plan), _P], _I),
    "qdt_bf16_linear": ([_P, _P, _P, _I64, _I64, _I64, _P, _I64, _P], _I),
    "qdt_w8a8_linear_noalloc": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _I64, _P], _I),
    "qdt_clock_record": ([_P, _I64], _I),
    "qdt_clock_record_used": ([C.POINTER(_I64)], _I),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res
    globals()[_name] = _fn

EXPORTED = tuple(_SIGS)


class QdtError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {qdt_status_string(status).decode()}")


def _check(status: int, where: str) -> None:
    if status != QDT_OK:
        raise QdtError(status, where)


def version() -> str:
    return qdt_version().decode()


def clock_record(buf: torch.Tensor | None) -> None:
    """Arm (int64 device tensor [entries, 4]) or disarm (None) the W8A8 GEMM clock record: each
    GEMM launch then fills one row per workgroup with its start / end shader-clock counter and
    100 MHz real-time counter, while rows remain."""
    if buf is None:
        _check(qdt_clock_record(None, 0), "qdt_clock_record")
        return
    _dev(buf, torch.int64, "buf")
    if buf.dim() != 2 or buf.shape[1] != 4 or not buf.is_contiguous():
        raise ValueError("clock record buffer must be a contiguous int64 [entries, 4] tensor")
    _check(qdt_clock_record(_ptr(buf), buf.shape[0]), "qdt_clock_record")


def clock_record_used() -> int:
    n = _I64(0)
    _check(qdt_clock_record_used(C.byref(n)), "qdt_clock_record_used")
    return n.value


# ------------------------------------------------------------------------------- helpers
def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _dev(t, dtype, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _rows(t, name):
    """(tensor, row stride) of a 2-D tensor with unit column stride."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    return t, t.stride(0)


# ------------------------------------------------------------------------------- torch API
def channel_absmax(X: torch.Tensor, s: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Calibration max-abs per column of bf16 X [M, K]; accumulates into ``s`` when given."""
    _dev(X, torch.bfloat16, "X")
    X, ldx = _rows(X, "X")
    M, K = X.shape
    acc = s is not None
    if s is None:
        s = torch.empty(K, dtype=torch.float32, device=X.device)
    _check(qdt_channel_absmax(_ptr(X), M, K, ldx, _ptr(s), int(acc), _stream(stream)), "qdt_channel_absmax")
    return s


def smooth_prepare(W: torch.Tensor, s: torch.Tensor | None, alpha: float = 0.5, stream=None):
    """Offline weight preparation.  Returns (Wq int8 [N,K], w_scale [N], inv_lambda [K], lambda [K])."""
    _dev(W, torch.bfloat16, "W")
    if not W.is_contiguous():
        raise ValueError("W must be contiguous")
    N, K = W.shape
    dev = W.device
    Wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    sw = torch.empty(N, dtype=torch.float32, device=dev)
    inv = torch.empty(K, dtype=torch.float32, device=dev)
    lam = torch.empty(K, dtype=torch.float32, device=dev)
    if s is not None:
        _dev(s, torch.float32, "s")
    _check(qdt_smooth_prepare(_ptr(W), _ptr(s), N, K, alpha, _ptr(Wq), _ptr(sw), _ptr(inv), _ptr(lam),
                              _stream(stream)), "qdt_smooth_prepare")
    return Wq, sw, inv, lam


def quantize_per_token(X: torch.Tensor, inv_lambda: torch.Tensor | None, Xq=None, x_scale=None, stream=None):
    """Per-token INT8 of bf16 X [M, K] (row stride may exceed K).  Returns (Xq int8 [M,K], x_scale [M])."""
    _dev(X, torch.bfloat16, "X")
    X, ldx = _rows(X, "X")
    M, K = X.shape
    if Xq is None:
        Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=X.device)
    _check(qdt_quantize_per_token(_ptr(X), _ptr(inv_lambda), M, K, ldx, _ptr(Xq), _ptr(x_scale), _stream(stream)),
           "qdt_quantize_per_token")
    return Xq, x_scale


def adaln_quantize(X: torch.Tensor, shift: torch.Tensor | None, scale: torch.Tensor | None,
                   inv_lambda: torch.Tensor | None, eps: float = 1e-6, Xq=None, x_scale=None, H=None,
                   want_h: bool = False, stream=None):
    """adaLN of bf16 X [M, K] (LayerNorm, * (1 + scale) + shift) fused with the per-token INT8 of
    the result for the next linear.  Returns (Xq, x_scale), or (Xq, x_scale, H) when ``want_h`` or
    ``H`` is given (H: bf16 [M, K], the modulated activations)."""
    _dev(X, torch.bfloat16, "X")
    X, ldx = _rows(X, "X")
    M, K = X.shape
    for t, n in ((shift, "shift"), (scale, "scale")):
        if t is not None:
            _dev(t, torch.bfloat16, n)
    if Xq is None:
        Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=X.device)
    if H is None and want_h:
        H = torch.empty((M, K), dtype=torch.bfloat16, device=X.device)
    _check(qdt_adaln_quantize(_ptr(X), ldx, _ptr(shift), _ptr(scale), float(eps), _ptr(inv_lambda), M, K, _ptr(Xq),
                              _ptr(x_scale), _ptr(H), _stream(stream)), "qdt_adaln_quantize")
    return (Xq, x_scale) if H is None else (Xq, x_scale, H)


def adaln_modulate(X: torch.Tensor, shift: torch.Tensor | None, scale: torch.Tensor | None, eps: float = 1e-6,
                   H=None, stream=None) -> torch.Tensor:
    """adaLN alone: bf16 H [M, K] = bf16(LayerNorm(X) * (1 + scale) + shift), for a bf16 consumer."""
    _dev(X, torch.bfloat16, "X")
    X, ldx = _rows(X, "X")
    M, K = X.shape
    if H is None:
        H = torch.empty((M, K), dtype=torch.bfloat16, device=X.device)
    _check(qdt_adaln_quantize(_ptr(X), ldx, _ptr(shift), _ptr(scale), float(eps), None, M, K, None, None, _ptr(H),
                              _stream(stream)), "qdt_adaln_quantize")
    return H


def mxfp4_quantize(X: torch.Tensor, colmul: torch.Tensor | None = None, Q=None, S=None, stream=None):
    """Block-scaled FP4 of bf16 X [M, K] (times colmul): (codes uint8 [M, K/2], biased block exponents
    uint8 [K/256, M, 8], stage-major: byte 2 (w % 4) + w / 4 of S[s, m] is block 8 s + w of row m)."""
    _dev(X, torch.bfloat16, "X")
    X, ldx = _rows(X, "X")
    M, K = X.shape
    if Q is None:
        Q = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    if S is None:
        S = torch.empty((K // 256, M, 8), dtype=torch.uint8, device=X.device)
    _check(qdt_mxfp4_quantize(_ptr(X), _ptr(colmul), M, K, ldx, _ptr(Q), _ptr(S), _stream(stream)),
           "qdt_mxfp4_quantize")
    return Q, S


_MX_EPI = {"bias": QDT_EPI_BIAS, "silu_gate": QDT_EPI_SILU_GATE, "head_rmsnorm": QDT_EPI_HEAD_RMSNORM,
           "acc_f32": QDT_EPI_ACC_F32}


def mxfp4_linear_plan(M: int, N: int, K: int, epilogue: str = "bias", tile: int | None = None,
                      split_k: int | None = None) -> dict:
    p = qdt_linear_plan()
    if tile is None and split_k is None:
        _check(qdt_mxfp4_linear_plan(M, N, K, _MX_EPI[epilogue], C.byref(p)), "qdt_mxfp4_linear_plan")
    else:
        _check(qdt_mxfp4_linear_plan_for(M, N, K, _MX_EPI[epilogue], QDT_TILE_AUTO if tile is None else tile,
                                         0 if split_k is None else split_k, C.byref(p)), "qdt_mxfp4_linear_plan_for")
    return p.as_dict()


def mxfp4_linear(Xq: torch.Tensor, Xs: torch.Tensor, Wq: torch.Tensor, Ws: torch.Tensor,
                 bias: torch.Tensor | None = None, epilogue: str = "bias", gamma=None, eps: float = 1e-6, out=None,
                 workspace=None, tile: int | None = None, split_k: int | None = None, stream=None) -> torch.Tensor:
    """Block-scaled FP4 linear: bf16 [M, N] = acc + bias ("bias"), bf16 [M, N/2] = silu(gate) * up
    ("silu_gate", W rows [gate; up]), RMSNorm of acc + bias over 256-wide heads with gamma
    ("head_rmsnorm"), or the fp32 accumulators ("acc_f32").
    Xq uint8 [M, K/2] and Xs uint8 [K/256, M, 8] from mxfp4_quantize of the activations; Wq, Ws the
    same of the weights.  ``tile`` / ``split_k`` force a plan (by default the library plans)."""
    for t, n in ((Xq, "Xq"), (Xs, "Xs"), (Wq, "Wq"), (Ws, "Ws")):
        _dev(t, torch.uint8, n)
    if bias is not None:
        _dev(bias, torch.bfloat16, "bias")
    M, N, K = Xq.shape[0], Wq.shape[0], Xq.shape[1] * 2
    if Wq.shape[1] * 2 != K or Xs.shape != (K // 256, M, 8) or Ws.shape != (K // 256, N, 8):
        raise ValueError("mxfp4_linear: inconsistent operand shapes")
    epi = _MX_EPI[epilogue]
    params = None
    if epi == QDT_EPI_HEAD_RMSNORM:
        if gamma is None:
            raise ValueError("head_rmsnorm needs gamma (bf16 [256])")
        _dev(gamma, torch.bfloat16, "gamma")
        params = qdt_rmsnorm_params(gamma.data_ptr(), 256, float(eps))
    if out is None:
        nout = N // 2 if epi == QDT_EPI_SILU_GATE else N
        out = torch.empty((M, nout), dtype=torch.float32 if epi == QDT_EPI_ACC_F32 else torch.bfloat16,
                          device=Xq.device)
    out, ldy = _rows(out, "out")
    planned = tile is not None or split_k is not None
    need = mxfp4_linear_plan(M, N, K, epilogue, tile, split_k)["workspace_bytes"]
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=Xq.device)
    args = [_ptr(Xq), _ptr(Xs), _ptr(Wq), _ptr(Ws), _ptr(bias), M, N, K, epi,
            None if params is None else C.cast(C.byref(params), C.c_void_p), _ptr(out), ldy,
            _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size()]
    if planned:
        plan = qdt_linear_plan()
        plan.tile = QDT_TILE_AUTO if tile is None else tile
        plan.split_k = 0 if split_k is None else split_k
        _check(qdt_mxfp4_linear_planned(*args, C.byref(plan), _stream(stream)), "qdt_mxfp4_linear_planned")
    else:
        _check(qdt_mxfp4_linear(*args, _stream(stream)), "qdt_mxfp4_linear")
    return out


QDT_WO_KSLICE = 8192


def wo_quantize(W: torch.Tensor, bits: int = 4, Wq=None, Wd=None, stream=None):
    """Weight-only blocks of bf16 W [N, K] (offline): codes (int8 [N, K] for 8 bits, uint8 [N, K/2]
    nibbles for 4 bits) and half-precision scale bits (int16 [N, K/32])."""
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    _dev(W, torch.bfloat16, "W")
    W, ldw = _rows(W, "W")
    N, K = W.shape
    if Wq is None:
        Wq = torch.empty((N, K if bits == 8 else K // 2), dtype=torch.int8 if bits == 8 else torch.uint8,
                         device=W.device)
    if Wd is None:
        Wd = torch.empty((N, K // 32), dtype=torch.int16, device=W.device)
    _check(qdt_wo_quantize(_ptr(W), N, K, ldw, bits, _ptr(Wq), _ptr(Wd), _stream(stream)), "qdt_wo_quantize")
    return Wq, Wd


def wo_linear_plan(M: int, N: int, K: int) -> dict:
    p = qdt_linear_plan()
    _check(qdt_wo_linear_plan(M, N, K, C.byref(p)), "qdt_wo_linear_plan")
    return p.as_dict()


def wo_linear(X: torch.Tensor, Wq: torch.Tensor, Wd: torch.Tensor, bias: torch.Tensor | None = None,
              epilogue: str = "bias", out=None, workspace=None, stream=None) -> torch.Tensor:
    """Weight-only linear: bf16 [M, N] = X . dequant(W)^T + bias ("bias"), or the fp32 accumulators
    ("acc_f32").  X bf16 [M, K]; Wq / Wd from wo_quantize (the code width gives the bit count).
    Every output row is bit-identical whatever M is."""
    _dev(X, torch.bfloat16, "X")
    X, ldx = _rows(X, "X")
    M, K = X.shape
    N = Wq.shape[0]
    if Wq.dtype == torch.int8 and Wq.shape == (N, K):
        bits = 8
    elif Wq.dtype == torch.uint8 and Wq.shape == (N, K // 2):
        bits = 4
    else:
        raise ValueError("wo_linear: Wq must be int8 [N, K] or uint8 [N, K/2]")
    _dev(Wd, torch.int16, "Wd")
    if Wd.shape != (N, K // 32):
        raise ValueError("wo_linear: Wd must be [N, K/32]")
    if bias is not None:
        _dev(bias, torch.bfloat16, "bias")
    if epilogue not in ("bias", "acc_f32"):
        raise ValueError("wo_linear: epilogue must be 'bias' or 'acc_f32'")
    epi = QDT_EPI_ACC_F32 if epilogue == "acc_f32" else QDT_EPI_BIAS
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32 if epilogue == "acc_f32" else torch.bfloat16, device=X.device)
    out, ldy = _rows(out, "out")
    need = wo_linear_plan(M, N, K)["workspace_bytes"]
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    _check(qdt_wo_linear(_ptr(X), ldx, _ptr(Wq), _ptr(Wd), bits, _ptr(bias), M, N, K, epi, _ptr(out), ldy,
                         _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
                         _stream(stream)), "qdt_wo_linear")
    return out

QDT_ATTN_HEAD_DIM = 256


def attention_workspace_size(S: int, H: int) -> int:
    n = _SZ(0)
    _check(qdt_attention_workspace_size(S, H, C.byref(n)), "qdt_attention_workspace_size")
    return n.value


def attention(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, heads: int, out=None, workspace=None,
              stream=None) -> torch.Tensor:
    """Softmax attention per 256-wide head: bf16 [S, 256 heads] = softmax(Q K^T / 16) V, head h in
    columns 256 h .. 256 h + 255.  Q, K, V: bf16 [S, ld] views with one common row stride (for
    example three column blocks of one fused projection output)."""
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _dev(t, torch.bfloat16, n)
    Q, ld = _rows(Q, "Q")
    K, ldk = _rows(K, "K")
    V, ldv = _rows(V, "V")
    if not (ld == ldk == ldv) or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("attention: Q, K, V must have the same shape and row stride")
    S = Q.shape[0]
    if Q.shape[1] < heads * QDT_ATTN_HEAD_DIM:
        raise ValueError("attention: fewer than 256 * heads columns")
    if out is None:
        out = torch.empty((S, heads * QDT_ATTN_HEAD_DIM), dtype=torch.bfloat16, device=Q.device)
    out, ldo = _rows(out, "out")
    need = attention_workspace_size(S, heads)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=Q.device)
    _check(qdt_attention(_ptr(Q), _ptr(K), _ptr(V), S, heads, ld, _ptr(out), ldo, _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream(stream)), "qdt_attention")
    return out

def linear_plan(M: int, N: int, K: int, epilogue: str = "bias", tile: int | None = None,
                split_k: int | None = None) -> dict:
    p = qdt_linear_plan()
    if tile is None and split_k is None:
        _check(qdt_w8a8_linear_plan(M, N, K, EPILOGUES[epilogue], C.byref(p)), "qdt_w8a8_linear_plan")
    else:
        _check(qdt_w8a8_linear_plan_for(M, N, K, EPILOGUES[epilogue], QDT_TILE_AUTO if tile is None else tile,
                                        0 if split_k is None else split_k, C.byref(p)), "qdt_w8a8_linear_plan_for")
    return p.as_dict()


def workspace_size(M: int, N: int, K: int, epilogue: str = "bias") -> int:
    b = C.c_size_t(0)
    _check(qdt_w8a8_linear_workspace_size(M, N, K, EPILOGUES[epilogue], C.byref(b)), "qdt_w8a8_linear_workspace_size")
    return int(b.value)


def w8a8_linear(Xq, x_scale, Wq, w_scale, bias=None, epilogue: str = "bias", gamma=None, head_dim: int = 256,
                eps: float = 1e-6, out=None, workspace=None, tile: int | None = None, split_k: int | None = None,
                stream=None):
    """W8A8 linear with a fused epilogue.  Returns bf16 [M, N_out] (int32 [M, N] for "acc_i32").

    ``tile`` / ``split_k`` force a plan (results are plan-independent); by default the
    library plans.  ``workspace`` is allocated here when the plan needs one and none is given.
    """
    epi = EPILOGUES[epilogue]
    M, K = Xq.shape
    N = Wq.shape[0]
    nout = N // 2 if epi == QDT_EPI_SILU_GATE else N
    dev = Xq.device
    if out is None:
        out = torch.empty((M, nout), dtype=torch.int32 if epi == QDT_EPI_ACC_I32 else torch.bfloat16, device=dev)
    params = None
    if epi == QDT_EPI_HEAD_RMSNORM:
        params = qdt_rmsnorm_params(gamma.data_ptr(), head_dim, eps)
    planned = tile is not None or split_k is not None
    if planned:
        plan = qdt_linear_plan()
        plan.tile = QDT_TILE_AUTO if tile is None else tile
        plan.split_k = 0 if split_k is None else split_k
        need = linear_plan(M, N, K, epilogue, tile, split_k)["workspace_bytes"]
    else:
        need = workspace_size(M, N, K, epilogue)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), _ptr(bias), M, N, K, epi,
            None if params is None else C.cast(C.byref(params), C.c_void_p), _ptr(out), out.stride(0),
            _ptr(workspace), wsb]
    if planned:
        _check(qdt_w8a8_linear_planned(*args, C.byref(plan), _stream(stream)), "qdt_w8a8_linear_planned")
    else:
        _check(qdt_w8a8_linear(*args, _stream(stream)), "qdt_w8a8_linear")
    return out


QDT_NOALLOC_SCRATCH_BYTES = 64 << 20


def w8a8_linear_noalloc(Xq, x_scale, Wq, w_scale, bias=None, epilogue: str = "bias", gamma=None,
                        head_dim: int = 256, eps: float = 1e-6, out=None, stream=None):
    """W8A8 linear that allocates nothing in the library: split-K partial sums go to the library's
    static per-device scratch (QDT_NOALLOC_SCRATCH_BYTES).  ``out`` is required, so this call
    allocates nothing either.  Calls on one device must not overlap in time."""
    if out is None:
        raise ValueError("w8a8_linear_noalloc needs a preallocated out")
    epi = EPILOGUES[epilogue]
    M, K = Xq.shape
    N = Wq.shape[0]
    params = None
    if epi == QDT_EPI_HEAD_RMSNORM:
        params = qdt_rmsnorm_params(gamma.data_ptr(), head_dim, eps)
    out, ldy = _rows(out, "out")
    _check(qdt_w8a8_linear_noalloc(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), _ptr(bias), M, N, K, epi,
                                   None if params is None else C.cast(C.byref(params), C.c_void_p), _ptr(out), ldy,
                                   _stream(stream)), "qdt_w8a8_linear_noalloc")
    return out


def bf16_linear(X, W, bias=None, out=None, stream=None):
    """bf16 linear of a protected layer: Y = X W^T + bias, fp32 accumulation on bf16 MFMA."""
    _dev(X, torch.bfloat16, "X")
    _dev(W, torch.bfloat16, "W")
    M, K = X.shape
    N = W.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _check(qdt_bf16_linear(_ptr(X), _ptr(W), _ptr(bias), M, N, K, _ptr(out), out.stride(0), _stream(stream)),
           "qdt_bf16_linear")
    return out


class PreparedLinear:
    """A W8A8 linear with its weights prepared once (offline) on the device."""

    def __init__(self, W: torch.Tensor, s: torch.Tensor | None, bias: torch.Tensor | None = None, alpha: float = 0.5):
        self.N, self.K = W.shape
        self.Wq, self.w_scale, self.inv_lambda, self.lam = smooth_prepare(W, s, alpha)
        self.bias = bias

    def __call__(self, X: torch.Tensor, epilogue: str = "bias", **kw) -> torch.Tensor:
        Xq, sx = quantize_per_token(X, self.inv_lambda)
        return w8a8_linear(Xq, sx, self.Wq, self.w_scale, self.bias, epilogue, **kw)
