"""Checks on the gfx950 assembly of the library's own device code (built
here from source, no GPU needed)."""

import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_wave_amd", "csrc")


def _device_asm(src: str) -> str:
    from mixture_experts_layer_wave_amd import build as B

    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "dev.s")
        cmd = [B.hipcc(), *B.HIPFLAGS, "--cuda-device-only", "-S", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            pytest.fail(f"hipcc -S failed on {src}:\n{r.stderr[-2000:]}")
        return open(out).read()


def test_m0_is_written_only_inside_the_copy_asm():
    """The weight-streaming kernels write M0 in inline assembly (the LDS
    address of a direct global-to-LDS copy).  M0 is reserved, so the asm
    cannot declare the write; the code is correct only while no compiler-
    generated instruction reads M0.  Every M0 reference must therefore sit
    inside an inline-asm block."""
    asm = _device_asm(os.path.join(CSRC, "decode.hip"))
    inside = False
    refs = 0
    for line in asm.splitlines():
        if ";;#ASMSTART" in line:
            inside = True
            continue
        if ";;#ASMEND" in line:
            inside = False
            continue
        code = line.split(";", 1)[0]
        if re.search(r"\bm0\b", code):
            refs += 1
            assert inside, f"M0 referenced outside the copy asm: {line.strip()}"
    assert refs > 0  # the copies themselves are there
