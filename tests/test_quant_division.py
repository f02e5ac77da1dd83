"""The quantize kernel's division for 16-bit weights, checked exhaustively on the CPU.

The kernel computes the quotient w/S with a reciprocal and one FMA correction instead of a
full IEEE division (see quant_pack.hip), and the scale's divisions by 15 and 7 the same way.  quotient_check.c enumerates every fp16 scale and
every bf16 (or fp16) weight pattern and requires the rounded quotient to equal the rounded
IEEE quotient wherever a group's weights can land.  A planted mistake (dropping the FMA
correction) must make the check fail, so the check itself is pinned.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "quotient_check.c")


def build(tmp_path, src_text=None):
    src = SRC
    if src_text is not None:
        src = str(tmp_path / "mutant.c")
        with open(src, "w") as fh:
            fh.write(src_text)
    exe = str(tmp_path / "quotient_check")
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", src, "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    return exe


pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


@pytest.mark.parametrize("mode,what", [(0, "bf16"), (1, "fp16")])
def test_fast_quotient_rounds_like_ieee_division(tmp_path, mode, what):
    exe = build(tmp_path)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    out = subprocess.run([exe, str(mode)], capture_output=True, text=True, timeout=600, env=env)
    assert out.returncode == 0, f"{what}: {out.stdout[-2000:]}"
    assert " bad 0" in out.stdout


def test_constant_divisions_equal_ieee(tmp_path):
    """s = range / 15 and s = max|w| / 7 via reciprocal and FMA correction, every fp32 input."""
    exe = build(tmp_path)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    out = subprocess.run([exe, "2"], capture_output=True, text=True, timeout=900, env=env)
    assert out.returncode == 0, out.stdout[-2000:]
    assert "bad 0" in out.stdout


def test_check_catches_a_missing_correction(tmp_path):
    text = open(SRC).read()
    planted = text.replace("const float q1 = fmaf(r, y, q0);", "const float q1 = q0 + 0.0f * r;")
    assert planted != text
    exe = build(tmp_path, planted)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    out = subprocess.run([exe, "0"], capture_output=True, text=True, timeout=600, env=env)
    assert out.returncode != 0
