"""The row loads of the quantizer kernels go out back to back.

A wave holds a row of X in registers, loaded as C 16-byte chunks per lane.  Written as a load under
a branch (zero for chunks past the row's end), some configurations compiled into a wait for all
outstanding loads right after each load, because the compiler copied the loaded value inside its
branch: the row's C loads then ran one after another, each paying the full memory latency (the
fused adaLN + quantize at 4608 x 4608 took 24.0 us that way against 21.0 us with the loads back to
back).  This check compiles qdt_quant.hip to gfx950 assembly with the library's flags and counts,
per kernel, the 16-byte global loads that are followed within two instructions by
`s_waitcnt vmcnt(0)`.  At most one is allowed (a row's last load may be waited for at once).  The
four-waves-per-row quantizer and the 16-waves-per-row one at K > 57344 keep such waits (their
branch form measured faster, or the clamped form spills) and are not checked."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from quantized_diffusion_transformer_amd import _build  # noqa: E402

KERNEL = re.compile(r"^(_ZN3qdt(?:17quant_rows_kernelILi(\d+)ELi(\d+)E|18adaln_quant_kernelILi(\d+)ELb([01])E)\S*):",
                    re.M)


def serialized_loads(fn_text):
    lines = [ln.split(";")[0].strip() for ln in fn_text.splitlines()]
    lines = [ln for ln in lines if ln and not ln.startswith(".") and not ln.endswith(":")]
    n = 0
    for i, ln in enumerate(lines):
        if ln.startswith("global_load_dwordx4 v["):
            if any(x.startswith("s_waitcnt") and "vmcnt(0)" in x for x in lines[i + 1:i + 3]):
                n += 1
    return n


def kernels(asm_text):
    """(name, wpr or None, chunks, text) of each quantizer / adaLN kernel in the assembly."""
    out = []
    ms = list(KERNEL.finditer(asm_text))
    for m in ms:
        end = asm_text.find(".Lfunc_end", m.end())
        text = asm_text[m.end():end]
        if m.group(2) is not None:
            out.append((m.group(1), int(m.group(2)), int(m.group(3)), text))
        else:
            out.append((m.group(1), None, int(m.group(4)), text))
    return out


def test_scanner_counts_a_wait_after_each_load():
    serial = ("global_load_dwordx4 v[2:5], v[0:1], off\n s_waitcnt vmcnt(0)\n v_mov_b32 v6, v3\n"
              "global_load_dwordx4 v[2:5], v[0:1], off offset:1024\n s_waitcnt vmcnt(0)\n")
    assert serialized_loads(serial) == 2
    back_to_back = ("global_load_dwordx4 v[2:5], v[0:1], off\n global_load_dwordx4 v[6:9], v[0:1], off offset:1024\n"
                    " v_mov_b32 v10, 0\n v_mov_b32 v11, 0\n s_waitcnt vmcnt(0)\n")
    assert serialized_loads(back_to_back) == 0


@pytest.fixture(scope="module")
def quant_asm(tmp_path_factory):
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path_factory.mktemp("asm") / "qdt_quant.s"
    cmd = [_build.hipcc(), *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
           os.path.join(_build.CSRC, "qdt_quant.hip"), "-o", str(out)]
    try:
        subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    except FileNotFoundError:
        pytest.skip("hipcc not found")
    return out.read_text()


def test_row_loads_back_to_back(quant_asm):
    ks = kernels(quant_asm)
    assert sum(1 for k in ks if k[1] is None) >= 14 and sum(1 for k in ks if k[1] is not None) >= 10
    bad = []
    for name, wpr, chunks, text in ks:
        if wpr == 4 or (wpr == 16 and chunks == 16):
            continue
        n = serialized_loads(text)
        if n > 1:
            bad.append(f"{name}: {n} loads each followed by a wait for all loads")
    assert not bad, "\n".join(bad)
