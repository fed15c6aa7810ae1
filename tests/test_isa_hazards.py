"""Inline-asm MFMAs are invisible to the compiler's hazard recognizer, which inserts the wait states
a VALU write needs before an MFMA reads the same registers only for the builtin forms.  This check
compiles each HIP source of the library to gfx950 assembly, with the library's own flags, and
asserts that no VALU instruction (v_accvgpr_mov and v_accvgpr_write included) writes a register
that an MFMA within the next HAZARD_WINDOW instructions reads as A, B or accumulator input.  The
window is counted in instructions, which never exceeds the wait states between them.  Such a write
one to three instructions ahead of an accumulating MFMA once broke the attention kernel's exact
results; the kernels now keep every such write at least four instructions away.

The other direction is checked too: an instruction other than an MFMA that reads the result
registers of an inline-asm MFMA (a VALU operand, an accumulator read, the data or address of an
LDS or global access) must come at least READ_AFTER_MFMA wait states after it.  That is more
than the largest read-after-MFMA-write requirement of the 16x16 MFMAs used here.  Wait states
are counted low: 1 per instruction, N + 1 per s_nop N, and only 4 per intervening MFMA, which
occupies the matrix pipeline for at least that long.  The attention loop relies on this distance
instead of a drain (the first read of the last scores is five MFMAs after them, in the next loop
iteration); the GEMMs drain with s_nop before reading accumulators.  The scan follows every path
of the control flow from each MFMA: fall-through, branch targets and loop back edges."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from quantized_diffusion_transformer_amd import _build  # noqa: E402

HAZARD_WINDOW = 3
READ_AFTER_MFMA = 19
SOURCES = ["qdt_gemm.hip", "qdt_wo.hip", "qdt_attn.hip"]


def _regs(op):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", op)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", op)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _instructions(asm_text):
    out = []
    for line in asm_text.splitlines():
        line = line.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        parts = line.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        out.append((parts[0], ops, line))
    return out


def hazards(asm_text, window=HAZARD_WINDOW):
    ins = _instructions(asm_text)
    found = []
    for i, (op, ops, line) in enumerate(ins):
        if not op.startswith("v_mfma") or len(ops) < 4:
            continue
        srcs = set().union(*(_regs(o) for o in ops[1:4]))
        for j in range(max(0, i - window), i):
            op2, ops2, line2 = ins[j]
            if op2.startswith("v_") and not op2.startswith("v_mfma") and ops2 and _regs(ops2[0]) & srcs:
                found.append(f"{line2}  ({i - j} before)  {line}")
    return found


def test_scanner_flags_a_close_write():
    """The scanner itself: a move into an accumulator right before the MFMA that reads it."""
    asm = "v_accvgpr_mov_b32 a72, a4\n v_mfma_f32_16x16x32_bf16 a[72:75], v[86:89], v[6:9], a[72:75]\n"
    assert len(hazards(asm)) == 1
    asm = ("v_mov_b32 v6, 0\n s_nop 0\n s_nop 0\n s_nop 0\n"
           " v_mfma_f32_16x16x32_bf16 a[72:75], v[86:89], v[6:9], a[72:75]\n")
    assert hazards(asm) == []


def _sources(op, ops):
    """Registers an instruction reads: every operand of a store, every operand but the first of
    anything else (the first is the destination)."""
    store = op.startswith(("ds_write", "ds_store", "global_store", "buffer_store", "flat_store", "scratch_store"))
    rd = ops if store else ops[1:]
    return set().union(*(_regs(o) for o in rd)) if rd else set()


def _wait_states(op, ops):
    if op == "s_nop":
        return int(ops[0], 0) + 1 if ops else 1
    if op.startswith("v_mfma"):
        return 4
    return 1


def _labels(asm_text):
    """Label -> index (in _instructions order) of the instruction that follows it."""
    out, n = {}, 0
    for line in asm_text.splitlines():
        line = line.split(";")[0].strip()
        if not line or line.startswith("."):
            if line.endswith(":") and line.startswith(".L"):
                out[line[:-1]] = n
            continue
        if line.endswith(":"):
            out[line[:-1]] = n
            continue
        n += 1
    return out


def _successors(j, op, ops, labels, n):
    if op in ("s_endpgm", "s_setpc_b64"):
        return []
    if op == "s_branch":
        return [labels[ops[0]]] if ops and ops[0] in labels else []
    if op.startswith("s_cbranch"):
        tgt = [labels[ops[0]]] if ops and ops[0] in labels else []
        return ([j + 1] if j + 1 < n else []) + tgt
    return [j + 1] if j + 1 < n else []


def read_after_mfma(asm_text, need=READ_AFTER_MFMA):
    """Reads of an MFMA's result registers by any other instruction fewer than `need` wait states
    after it, along every path of the control flow (fall-through, branches, loop back edges)."""
    ins = _instructions(asm_text)
    labels = _labels(asm_text)
    found = []
    for i, (op, ops, line) in enumerate(ins):
        if not op.startswith("v_mfma") or len(ops) < 4:
            continue
        dst = _regs(ops[0])
        best = {}
        work = [(j, 0) for j in _successors(i, op, ops, labels, len(ins))]
        hit = None
        while work and hit is None:
            j, ws = work.pop()
            if ws >= need or best.get(j, need) <= ws:
                continue
            best[j] = ws
            op2, ops2, line2 = ins[j]
            if not op2.startswith("v_mfma") and _sources(op2, ops2) & dst:
                hit = f"{line}  ->  {line2}  ({ws} wait states)"
                break
            if op2.startswith("v_") and not op2.startswith("v_mfma") and ops2 and _regs(ops2[0]) & dst:
                continue  # overwritten before any read on this path
            for k in _successors(j, op2, ops2, labels, len(ins)):
                work.append((k, ws + _wait_states(op2, ops2)))
        if hit:
            found.append(hit)
    return found


def test_scanner_flags_a_close_read():
    """The scanner itself: reading an MFMA result after too few wait states, and after enough."""
    mf = "v_mfma_f32_16x16x32_bf16 a[0:3], v[86:89], v[6:9], a[0:3]\n"
    other = "v_mfma_f32_16x16x32_bf16 a[4:7], v[86:89], v[6:9], a[4:7]\n"
    assert len(read_after_mfma(mf + other * 2 + "v_accvgpr_read_b32 v1, a2\n")) == 1
    assert len(read_after_mfma(mf + " s_nop 7\n" + "global_store_dwordx4 v[2:3], a[0:3], off\n")) == 1
    assert read_after_mfma(mf + other * 5 + "v_accvgpr_read_b32 v1, a2\n") == []
    assert read_after_mfma(mf + " s_nop 7\n s_nop 7\n s_nop 2\n v_accvgpr_read_b32 v1, a2\n") == []
    # another MFMA chaining on the accumulator is not a read by another unit
    assert read_after_mfma(mf + mf + " s_nop 7\n s_nop 7\n s_nop 7\n") == []
    # a read at the top of a loop, reached from an MFMA at its bottom through the back edge
    loop = (".LBB0_1:\n v_accvgpr_read_b32 v1, a2\n s_nop 7\n s_nop 7\n s_nop 7\n" + mf +
            " s_cbranch_scc1 .LBB0_1\n s_endpgm\n")
    assert len(read_after_mfma(loop)) == 1


def _asm(src, tmp_path):
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / (src + ".s")
    cmd = [_build.hipcc(), *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
           os.path.join(_build.CSRC, src), "-o", str(out)]
    try:
        subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    except FileNotFoundError:
        pytest.skip("hipcc not found")
    return out.read_text()


@pytest.fixture(scope="module")
def asm_texts(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    return {src: _asm(src, d) for src in SOURCES}


@pytest.mark.parametrize("src", SOURCES)
def test_no_valu_write_next_to_an_mfma_read(src, asm_texts):
    found = hazards(asm_texts[src])
    assert not found, "\n".join(found[:10])


@pytest.mark.parametrize("src", SOURCES)
def test_no_read_of_an_mfma_result_too_soon(src, asm_texts):
    found = read_after_mfma(asm_texts[src])
    assert not found, "\n".join(found[:10])
