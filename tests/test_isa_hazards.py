"""The LDS-DMA loads are inline asm, which the compiler's hazard checks do not see: each
one must carry its own wait states (s_nop 4 right before the load) so that an SGPR
operand written by a VALU instruction, or M0 written by an SALU instruction, is read
correctly.  This compiles every kernel source that issues such loads to gfx950 assembly
and checks the instruction before each load."""
import os
import re
import subprocess

import pytest

from mixture_experts_routed_topk_amd import build_lib

CSRC = build_lib.CSRC


def _dma_sources():
    out = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip") and "dma_lds_" in open(os.path.join(CSRC, f)).read():
            out.append(f)
    return out


@pytest.mark.skipif(not os.path.exists(build_lib.HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", _dma_sources())
def test_lds_dma_loads_carry_wait_states(src, tmp_path):
    asm = tmp_path / (src + ".s")
    cmd = [build_lib.HIPCC, *build_lib.FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(asm)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    ins = []
    for line in open(asm):
        t = line.strip()
        if not t or t.startswith((";", ".", "//")) or t.endswith(":"):
            continue
        ins.append(t)
    loads = [i for i, t in enumerate(ins) if t.startswith("global_load_lds")]
    assert loads, "no LDS DMA loads found"
    for i in loads:
        m = re.match(r"s_nop\s+(\d+)", ins[i - 1])
        assert m and int(m.group(1)) >= 4, f"{src}: '{ins[i]}' is preceded by '{ins[i - 1]}'"
