"""Host-side checks of the kernels' LDS layouts (tests/layout_check.hip, compiled for the host only with
hipcc and run on the CPU): the K/V block image is injective and in bounds, and the operand reads of the INT4
kernel and the FP16 kernel's V^T reads are free of LDS bank conflicts under a 64-bank model (which flags the
unpermuted layout). No GPU needed."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_lds_layouts(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = tmp_path / "layout_check"
    cmd = [hipcc, "-O1", "--offload-arch=gfx950", "--offload-host-only", "-std=c++17",
           "-I", os.path.join(ROOT, "int4_quantized_flashattention_amd", "csrc"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "layout_check.hip"), "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout
