"""Host check of the exact-division identities the bulk write kernel relies
on (reciprocal with one Markstein correction; corrected hardware
reciprocal), exhaustive over the binary32 significands of the dividend and
the bfloat16 significands of the divisor.  Runs the C check in
tests/csrc/div_exact.c, built with gcc and contraction disabled."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_division_identities_exhaustive(tmp_path):
    exe = tmp_path / "div_exact"
    src = os.path.join(HERE, "csrc", "div_exact.c")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", str(exe), src, "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "division mismatches 0" in r.stdout and "reciprocal mismatches 0" in r.stdout
