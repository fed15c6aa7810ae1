"""Host-side tests of the C ABI (no GPU): exported symbols, validation errors, planner.

Every call here fails validation or is a pure host computation, so nothing reaches HIP.
"""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

qdt = pytest.importorskip("quantized_diffusion_transformer_amd")

P = C.c_void_p


def header_functions():
    text = open(os.path.join(ROOT, "include", "qdt.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qdt_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    declared = header_functions()
    assert len(declared) >= 10
    lib = C.CDLL(qdt.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in qdt.h but not exported"
    assert sorted(qdt.EXPORTED) == declared


def test_status_strings_and_version():
    for s in range(8):
        assert qdt.qdt_status_string(s).decode().startswith("QDT_")
    assert "gfx950" in qdt.version()


def A(addr=0x10000):
    return P(addr)


def test_quantize_validation():
    f = qdt.qdt_quantize_per_token
    assert f(A(), None, 4, 100, 100, A(0x20000), A(0x30000), None) == qdt.QDT_ESHAPE  # K % 64
    assert f(A(), None, 4, 128, 64, A(0x20000), A(0x30000), None) == qdt.QDT_ESHAPE   # ldx < K
    assert f(A(), None, -1, 128, 128, A(0x20000), A(0x30000), None) == qdt.QDT_ESHAPE
    assert f(None, None, 4, 128, 128, A(0x20000), A(0x30000), None) == qdt.QDT_EINVAL
    assert f(A(0x10008), None, 4, 128, 128, A(0x20000), A(0x30000), None) == qdt.QDT_EALIGN
    assert f(A(), None, 4, 128, 132, A(0x20000), A(0x30000), None) == qdt.QDT_EALIGN   # row stride
    assert f(A(), None, 4, 128, 128, A(0x10100), A(0x30000), None) == qdt.QDT_EALIAS   # Xq inside X
    assert f(A(), None, 4, qdt.QDT_MAX_K + 64, qdt.QDT_MAX_K + 64, A(0x2000000), A(0x3000000), None) == qdt.QDT_ESHAPE
    assert f(A(), None, 0, 128, 128, A(0x20000), A(0x30000), None) == qdt.QDT_OK        # M = 0: no-op


def test_adaln_quantize_validation():
    f = qdt.qdt_adaln_quantize
    outs = (A(0x200000), A(0x300000), A(0x400000))              # Xq, x_scale, H

    def call(X=A(), ldx=128, shift=None, scale=None, eps=1e-6, inv=None, M=4, K=128, outs=outs):
        return f(X, ldx, shift, scale, eps, inv, M, K, *outs, None)
    assert call(K=100, ldx=100) == qdt.QDT_ESHAPE                      # K % 64
    assert call(K=qdt.QDT_MAX_ADALN_K + 64, ldx=qdt.QDT_MAX_ADALN_K + 64,
                outs=(A(0x2000000), A(0x3000000), None)) == qdt.QDT_ESHAPE  # one wave holds a row
    assert call(ldx=64) == qdt.QDT_ESHAPE
    assert call(M=-1) == qdt.QDT_ESHAPE
    assert call(eps=0.0) == qdt.QDT_EINVAL
    assert call(eps=float("nan")) == qdt.QDT_EINVAL
    assert call(eps=float("inf")) == qdt.QDT_EINVAL
    assert call(X=None) == qdt.QDT_EINVAL
    assert call(X=A(0x10008)) == qdt.QDT_EALIGN
    assert call(shift=A(0x500004)) == qdt.QDT_EALIGN
    assert call(ldx=132) == qdt.QDT_EALIGN
    assert call(outs=(A(0x10100), A(0x300000), None)) == qdt.QDT_EALIAS           # Xq inside X
    assert call(outs=(A(0x200000), A(0x300000), A(0x200100))) == qdt.QDT_EALIAS    # H over Xq
    assert call(inv=A(0x300000)) == qdt.QDT_EALIAS                                 # x_scale over inv_lambda
    assert call(outs=(A(0x200000), None, A(0x400000))) == qdt.QDT_EINVAL           # Xq without x_scale
    assert call(outs=(None, None, None)) == qdt.QDT_EINVAL                        # nothing to write
    assert call(M=0) == qdt.QDT_OK


def test_mxfp4_validation():
    q = qdt.qdt_mxfp4_quantize
    assert q(A(), None, 4, 128, 128, A(0x200000), A(0x300000), None) == qdt.QDT_ESHAPE    # K % 256 (stages)
    assert q(A(), None, 4, 256, 128, A(0x200000), A(0x300000), None) == qdt.QDT_ESHAPE     # ldx < K
    assert q(A(), None, 4, 256, 256, A(0x200008), A(0x300000), None) == qdt.QDT_EALIGN
    assert q(A(), None, 4, 256, 256, A(0x10010), A(0x300000), None) == qdt.QDT_EALIAS     # Q inside X
    assert q(A(), None, 4, 256, 256, None, A(0x300000), None) == qdt.QDT_EINVAL
    assert q(A(), None, 0, 256, 256, A(0x200000), A(0x300000), None) == qdt.QDT_OK
    f = qdt.qdt_mxfp4_linear

    def lin(M=64, N=128, K=256, epi=0, Y=0x900000, ldy=None, xs=0x200000, ws=0x400000):
        return f(A(0x100000), A(xs), A(0x300000), A(ws), None, M, N, K, epi, None, A(Y), N if ldy is None else ldy,
                 None, 0, None)
    assert lin(K=128) == qdt.QDT_ESHAPE                 # whole 256-element stages
    assert lin(N=120) == qdt.QDT_ESHAPE
    assert lin(epi=2, N=512) == qdt.QDT_EINVAL          # head RMSNorm without its parameters
    assert lin(epi=2, N=384) == qdt.QDT_ESHAPE          # whole 256-column heads
    assert lin(epi=3) == qdt.QDT_EINVAL                 # int32 accumulators are the W8A8 linear's
    assert lin(epi=1, N=48) == qdt.QDT_ESHAPE           # gate and up halves of whole 16-row fragments
    assert lin(epi=1, N=128, ldy=32) == qdt.QDT_ESHAPE  # ldy >= F = N / 2
    assert lin(ldy=64) == qdt.QDT_ESHAPE
    assert lin(xs=0x200002) == qdt.QDT_EALIGN           # exponent rows read as dwords
    assert lin(Y=0x300000 + 64) == qdt.QDT_EALIAS        # Y over Wq
    assert lin(M=0) == qdt.QDT_OK
    # deep K with few output tiles splits K and needs a workspace for the fp32 partials
    p = qdt.mxfp4_linear_plan(512, 4608, 53248)
    assert p["split_k"] > 1 and p["tile_m"] == 256 and p["workspace_bytes"] == p["split_k"] * 512 * 4608 * 4
    big = 0x10000000000
    assert f(A(big), A(2 * big), A(3 * big), A(4 * big), None, 512, 4608, 53248, 0, None, A(5 * big), 4608,
             None, 0, None) == qdt.QDT_EWORKSPACE
    assert qdt.mxfp4_linear_plan(4608, 4608, 4608)["split_k"] == 1


def test_mxfp4_planner():
    # 4608^3: 256 tiles of 288 x 288, one round on 256 compute units (324 tiles of 256 x 256 need two)
    p = qdt.mxfp4_linear_plan(4608, 4608, 4608)
    assert (p["tile_m"], p["tile_n"], p["grid"], p["split_k"]) == (288, 288, 256, 1)
    # gated SiLU and head RMSNorm need 256 weight rows per tile; 288 x 256 only on request
    assert qdt.mxfp4_linear_plan(4608, 24576, 4608, "silu_gate")["tile_n"] == 256
    p = qdt.mxfp4_linear_plan(4608, 24576, 4608, "silu_gate", tile=qdt.QDT_TILE_288x256)
    assert (p["tile_m"], p["tile_n"], p["tiles_n"]) == (288, 256, 96)
    p = qdt.mxfp4_linear_plan(16896, 4608, 4608, "head_rmsnorm", tile=qdt.QDT_TILE_288x256)
    assert (p["tile_m"], p["tile_n"], p["tiles_m"]) == (288, 256, 59)
    with pytest.raises(qdt.QdtError):   # 288 x 288 has no 256-column head
        qdt.mxfp4_linear_plan(4608, 4608, 4608, "head_rmsnorm", tile=qdt.QDT_TILE_288)
    with pytest.raises(qdt.QdtError):   # 224 x 256 is an int8 tile
        qdt.mxfp4_linear_plan(4608, 4608, 4608, tile=qdt.QDT_TILE_224x256)
    # a forced K split
    p = qdt.mxfp4_linear_plan(600, 1024, 8192, tile=qdt.QDT_TILE_288, split_k=4)
    assert p["tile_m"] == 288 and p["split_k"] == 4 and p["workspace_bytes"] == 4 * 600 * 1024 * 4


def test_weight_only_validation():
    q = qdt.qdt_wo_quantize
    assert q(A(), 16, 64, 64, 3, A(0x200000), A(0x300000), None) == qdt.QDT_EINVAL       # bits 4 or 8
    assert q(A(), 16, 48, 48, 4, A(0x200000), A(0x300000), None) == qdt.QDT_ESHAPE       # K % 32
    assert q(A(), 16, 64, 32, 4, A(0x200000), A(0x300000), None) == qdt.QDT_ESHAPE       # ldw < K
    assert q(A(), 16, 64, 68, 4, A(0x200000), A(0x300000), None) == qdt.QDT_EALIGN       # ldw % 8
    assert q(A(), 16, 64, 64, 8, A(0x200008), A(0x300000), None) == qdt.QDT_EALIGN       # Wq 16 bytes
    assert q(A(), 16, 64, 64, 8, A(0x200000), A(0x300001), None) == qdt.QDT_EALIGN       # Wd 2 bytes
    assert q(A(), 16, 64, 64, 8, A(0x10000 + 64), A(0x300000), None) == qdt.QDT_EALIAS   # Wq over W
    assert q(A(), 16, 64, 64, 8, None, A(0x300000), None) == qdt.QDT_EINVAL
    assert q(A(), 0, 64, 64, 8, A(0x200000), A(0x300000), None) == qdt.QDT_OK
    f = qdt.qdt_wo_linear

    def lin(M=64, N=128, K=512, bits=4, epi=0, Y=0x900000, ldy=None, ldx=None, wd=0x400000, ws=None, wsb=0):
        return f(A(0x100000), K if ldx is None else ldx, A(0x300000), A(wd), bits, None, M, N, K, epi, A(Y),
                 N if ldy is None else ldy, None if ws is None else A(ws), wsb, None)
    assert lin(bits=6) == qdt.QDT_EINVAL
    assert lin(epi=1) == qdt.QDT_EINVAL                 # bias or fp32 accumulators only
    assert lin(epi=3) == qdt.QDT_EINVAL
    assert lin(K=256) == qdt.QDT_ESHAPE                 # stages in fours: K % 512
    assert lin(N=120) == qdt.QDT_ESHAPE
    assert lin(ldx=256) == qdt.QDT_ESHAPE
    assert lin(ldy=64) == qdt.QDT_ESHAPE
    assert lin(ldx=516) == qdt.QDT_EALIGN
    assert lin(wd=0x400001) == qdt.QDT_EALIGN
    assert lin(Y=0x300000 + 64) == qdt.QDT_EALIAS        # Y over Wq
    assert lin(M=0) == qdt.QDT_OK
    # the K slicing is fixed: the same split for every row count
    plans = [qdt.wo_linear_plan(M, 4608, 53248) for M in (1, 512, 4608, 100000)]
    assert {p["split_k"] for p in plans} == {7} and all(p["tile_m"] == 256 for p in plans)
    assert plans[1]["workspace_bytes"] == 7 * 512 * 4608 * 4 and plans[1]["grid"] == 2 * 18 * 7
    assert qdt.wo_linear_plan(300, 4608, 8192)["split_k"] == 1
    assert qdt.wo_linear_plan(300, 4608, 8704)["split_k"] == 2
    big = 0x10000000000
    assert f(A(big), 53248, A(2 * big), A(3 * big), 4, None, 512, 4608, 53248, 0, A(5 * big), 4608, None, 0,
             None) == qdt.QDT_EWORKSPACE
    assert f(A(big), 53248, A(2 * big), A(3 * big), 4, None, 512, 4608, 53248, 0, A(5 * big), 4608, A(6 * big),
             7 * 512 * 4608 * 4 - 16, None) == qdt.QDT_EWORKSPACE

def test_attention_validation():
    f = qdt.qdt_attention
    # up to 8192 tokens V is read transposed in LDS (no V^T region): 16 bytes of rerun flags per
    # workgroup (one int per wave), plus the pieces' fp32 outputs when the last round is split
    n = qdt.attention_workspace_size(100, 2)
    assert n == 2 * 16 and qdt.attention_workspace_size(256, 1) == 16
    # 4608 tokens x 18 heads: 324 (query block, head) tiles, 68 past one round of 256, each split
    # into 3 key ranges: 460 workgroups' rerun flags and 204 pieces' fp32 outputs
    assert qdt.attention_workspace_size(4608, 18) == 460 * 16 + 204 * 256 * 258 * 4
    # 8192 tokens still reads V transposed; 8193 writes V^T first (keys padded to 8224)
    assert qdt.attention_workspace_size(8192, 1) == 32 * 16
    assert qdt.attention_workspace_size(8193, 1) == 256 * 8224 * 2 + 33 * 16
    # 16896 x 18: 1188 tiles, 164 past four rounds, more than half a round: no split
    assert qdt.attention_workspace_size(16896, 18) == 18 * 256 * 16896 * 2 + 1188 * 16
    # 2048 x 40: 320 tiles, 64 past one round, 4 key ranges each
    assert qdt.attention_workspace_size(2048, 40) == 512 * 16 + 256 * 256 * 258 * 4

    def att(S=100, H=2, ld=512, ldo=512, O=0x900000, ws=0x2000000, wsb=None, q=0x100000):
        return f(A(q), A(0x300000), A(0x500000), S, H, ld, A(O), ldo, A(ws), n if wsb is None else wsb, None)
    assert att(H=0) == qdt.QDT_ESHAPE
    assert att(S=-1) == qdt.QDT_ESHAPE
    assert att(ld=500) == qdt.QDT_ESHAPE                 # fewer than 256 H columns
    assert att(ldo=256) == qdt.QDT_ESHAPE
    assert att(ld=516) == qdt.QDT_EALIGN
    assert att(q=0x100008) == qdt.QDT_EALIGN
    assert att(wsb=n - 16) == qdt.QDT_EWORKSPACE
    assert att(O=0x300000 + 1024) == qdt.QDT_EALIAS      # O over K
    assert att(ws=0x500000 + 64) == qdt.QDT_EALIAS       # workspace over V
    assert att(S=0) == qdt.QDT_OK

def test_smooth_prepare_validation():
    f = qdt.qdt_smooth_prepare
    outs = (A(0x100000), A(0x200000), A(0x300000), A(0x400000))
    assert f(A(), None, 8, 100, 0.5, *outs, None) == qdt.QDT_ESHAPE
    assert f(A(), None, 8, 128, 1.5, *outs, None) == qdt.QDT_EINVAL
    assert f(A(), None, 8, 128, float("nan"), *outs, None) == qdt.QDT_EINVAL
    assert f(A(), None, 8, 128, 0.5, A(0x100000), A(0x200000), None, A(0x400000), None) == qdt.QDT_EINVAL
    assert f(A(), None, 8, 128, 0.5, A(0x10010), A(0x200000), A(0x300000), A(0x400000), None) == qdt.QDT_EALIAS
    assert f(A(), None, 8, 128, 0.5, A(0x100000), A(0x100000), A(0x300000), A(0x400000), None) == qdt.QDT_EALIAS


def _lin(M=64, N=128, K=256, epi=0, params=None, Y=0x900000, ldy=None, ws=None, wsb=0, bias=None,
         xq=0x100000, sx=0x200000, wq=0x300000, sw=0x400000):
    ldy = (N // 2 if epi == 1 else N) if ldy is None else ldy
    return qdt.qdt_w8a8_linear(A(xq), A(sx), A(wq), A(sw), None if bias is None else A(bias), M, N, K, epi, params,
                               A(Y), ldy, None if ws is None else A(ws), wsb, None)


def test_linear_validation():
    assert _lin(K=100) == qdt.QDT_ESHAPE
    assert _lin(K=192) == qdt.QDT_ESHAPE                           # INT8 GEMM stages are 128 bytes of K
    assert _lin(N=120) == qdt.QDT_ESHAPE
    assert _lin(N=48, epi=1) == qdt.QDT_ESHAPE                     # SILU needs N % 32
    assert _lin(N=384, epi=2, params=None) == qdt.QDT_ESHAPE        # heads need N % 256
    assert _lin(N=512, epi=2, params=None) == qdt.QDT_EINVAL        # missing gamma
    bad = qdt.qdt_rmsnorm_params(0x500000, 128, 1e-6)
    assert _lin(N=512, epi=2, params=C.cast(C.byref(bad), P)) == qdt.QDT_ESHAPE
    neg = qdt.qdt_rmsnorm_params(0x500000, 256, -1.0)
    assert _lin(N=512, epi=2, params=C.cast(C.byref(neg), P)) == qdt.QDT_EINVAL
    assert _lin(epi=7) == qdt.QDT_EINVAL
    assert _lin(ldy=64) == qdt.QDT_ESHAPE
    assert _lin(ldy=132) == qdt.QDT_EALIGN
    assert _lin(Y=0x900008) == qdt.QDT_EALIGN
    assert _lin(Y=0x300000 + 1024) == qdt.QDT_EALIAS                # Y over Wq
    assert _lin(M=0) == qdt.QDT_OK                                   # empty: nothing to do


def test_linear_workspace_checks():
    M, N, K = 512, 4608, 53248
    need = qdt.workspace_size(M, N, K)
    plan = qdt.linear_plan(M, N, K)
    assert plan["split_k"] > 1 and need == plan["split_k"] * M * N * 4
    big = 0x10000000000
    args = dict(M=M, N=N, K=K, xq=big, sx=2 * big, wq=3 * big, sw=4 * big, Y=5 * big)
    assert _lin(**args) == qdt.QDT_EWORKSPACE
    assert _lin(ws=6 * big, wsb=need - 16, **args) == qdt.QDT_EWORKSPACE
    assert _lin(ws=5 * big + 64, wsb=need, **args) == qdt.QDT_EALIAS  # workspace over Y


def test_bf16_linear_validation():
    f = qdt.qdt_bf16_linear
    assert f(A(), A(0x200000), None, 4, 100, 128, A(0x900000), 100, None) == qdt.QDT_ESHAPE
    assert f(A(), A(0x200000), None, 4, 128, 96, A(0x900000), 128, None) == qdt.QDT_ESHAPE
    assert f(A(), A(0x200000), None, 4, 128, 128, A(0x10000), 128, None) == qdt.QDT_EALIAS
    assert f(A(), A(0x200000), None, 0, 128, 128, A(0x900000), 128, None) == qdt.QDT_OK


@pytest.mark.parametrize("M,N,K,epi,tm,tn,split", [
    (4608, 4608, 4608, "bias", 288, 288, 1),          # attention projection: 256 tiles of 288 x 288
    (512, 4608, 53248, "bias", 256, 256, 7),          # deep-K text projection: split K over 7 slices
    (4608, 4608, 53248, "bias", 288, 288, 1),         # its zero-padded variant fills the GPU without a split
    (16896, 4608, 4608, "head_rmsnorm", 256, 256, 1),  # heads need 256-wide tiles
    (6037, 4608, 4608, "head_rmsnorm", 224, 256, 1),  # 486 tiles of 224 x 256: two full rounds
    (4608, 24576, 4608, "silu_gate", 256, 256, 1),
    (64, 128, 256, "bias", 224, 256, 1),            # one partial tile: the smallest that holds it
])
def test_planner_choices(M, N, K, epi, tm, tn, split):
    p = qdt.linear_plan(M, N, K, epi)
    assert p["tile_m"] == tm and p["tile_n"] == tn and p["split_k"] == split
    nout_tiles = -(-(N // 2) // (tn // 2)) if epi == "silu_gate" else -(-N // tn)
    assert p["tiles_m"] == -(-M // tm) and p["tiles_n"] == nout_tiles
    assert p["grid"] == p["tiles_m"] * p["tiles_n"] * p["split_k"]
    assert p["workspace_bytes"] == (split * M * N * 4 if split > 1 else 0)


def test_plan_for_honours_requests():
    p = qdt.linear_plan(600, 1024, 4096, "bias", tile=qdt.QDT_TILE_288, split_k=5)
    assert p["tile_m"] == 288 and p["split_k"] == 5 and p["k_tiles"] == 32  # 128-byte K stages
    # a request that would leave an empty slice is rounded down
    p = qdt.linear_plan(600, 1024, 256, "bias", split_k=3)
    assert p["split_k"] == 2
    with pytest.raises(qdt.QdtError):
        qdt.linear_plan(600, 1024, 4096, "head_rmsnorm", tile=qdt.QDT_TILE_288)
    p = qdt.linear_plan(600, 1024, 4096, "head_rmsnorm", tile=qdt.QDT_TILE_288x256)
    assert p["tile_m"] == 288 and p["tile_n"] == 256
    p = qdt.linear_plan(600, 1024, 4096, "silu_gate", tile=qdt.QDT_TILE_224x256)
    assert p["tile_m"] == 224 and p["tile_n"] == 256
    with pytest.raises(qdt.QdtError):
        qdt.linear_plan(600, 1024, 4096, "bias", tile=4)


def test_noalloc_linear_validation():
    f = qdt.qdt_w8a8_linear_noalloc
    # 512 x 11008 x 53248 splits K 3 ways: 67.6 MB of partial sums, more than the static scratch;
    # refused right after planning, before any pointer is looked at
    M, N, K = 512, 11008, 53248
    assert qdt.linear_plan(M, N, K, "bias")["workspace_bytes"] > qdt.QDT_NOALLOC_SCRATCH_BYTES
    assert f(None, None, None, None, None, M, N, K, qdt.QDT_EPI_BIAS, None, None, N, None) == qdt.QDT_EWORKSPACE
    # the usual argument checks, as qdt_w8a8_linear
    assert f(A(), A(0x20000), A(0x30000), A(0x40000), None, 4, 16, 64, qdt.QDT_EPI_BIAS, None, A(0x50000), 16,
             None) == qdt.QDT_ESHAPE                                                    # K % 128
    assert f(A(), A(0x20000), A(0x30000), A(0x40000), None, 4, 16, 128, 9, None, A(0x50000), 16,
             None) == qdt.QDT_EINVAL                                                    # epilogue
    assert f(A(), A(0x20000), A(0x30000), A(0x40000), None, 4, 16, 128, qdt.QDT_EPI_BIAS, None, A(0x10040), 16,
             None) == qdt.QDT_EALIAS                                                    # Y inside Xq
    assert f(None, None, None, None, None, 0, 16, 128, qdt.QDT_EPI_BIAS, None, None, 16, None) == qdt.QDT_OK
