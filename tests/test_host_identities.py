"""Host checks of arithmetic identities used inside the device kernels (no
GPU): each is a statement about IEEE binary32 arithmetic, checked over every
input it is applied to."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_division_by_six_with_one_fma_correction_is_exact(tmp_path):
    """The block-scale step amax_b / 6 runs as a multiply by RN(1/6) plus one
    fma correction for amax_b in [2^-125, FLT_MAX]; every such binary32 value
    must give the correctly rounded quotient."""
    exe = tmp_path / "div6"
    src = os.path.join(HERE, "host_div6_identity.c")
    r = subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", src, "-o",
                        str(exe), "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("gcc unavailable: " + r.stderr[:200])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600,
                         env=dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1))))
    assert out.returncode == 0
    assert out.stdout.strip() == "0"
