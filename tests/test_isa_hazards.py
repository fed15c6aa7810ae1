"""Inline-asm MFMAs are invisible to the compiler's hazard recognizer, which inserts the wait states
a VALU write needs before an MFMA reads the same registers only for the builtin forms.  This check
compiles each HIP source of the library to gfx950 assembly, with the library's own flags, and
asserts that no VALU instruction (v_accvgpr_mov and v_accvgpr_write included) writes a register
that an MFMA within the next HAZARD_WINDOW instructions reads as A, B or accumulator input.  The
window is counted in instructions, which never exceeds the wait states between them.  Such a write
one to three instructions ahead of an accumulating MFMA once broke the attention kernel's exact
results; the kernels now keep every such write at least four instructions away."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from quantized_diffusion_transformer_amd import _build  # noqa: E402

HAZARD_WINDOW = 3
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


@pytest.mark.parametrize("src", SOURCES)
def test_no_valu_write_next_to_an_mfma_read(src, tmp_path):
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / (src + ".s")
    cmd = [_build.hipcc(), *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
           os.path.join(_build.CSRC, src), "-o", str(out)]
    try:
        subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    except FileNotFoundError:
        pytest.skip("hipcc not found")
    found = hazards(out.read_text())
    assert not found, "\n".join(found[:10])
