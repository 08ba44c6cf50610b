"""The NVFP4 append kernels decide each element's e2m1 magnitude in fp32
(three fused multiply-adds in a binary search over the decision points)
when the tensor scale S lies in [2^-109, 2^100], and in fp64 otherwise.  The
fp32 decisions are exact there: t e4m3 is exact in fp32, and a - (t e4m3) S,
rounded once by the fused multiply-add, is zero only when the exact
difference is (a nonzero difference is at least 2^-143 in magnitude).  This
compiles a host C check (tests/nvfp4_host/) that compares both decisions on
about 7e7 (magnitude, block scale, tensor scale) triples, decision-point
neighbours included.  No GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fp32_decisions_equal_the_fp64_ones(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    exe = tmp_path / "f32_decisions"
    src = os.path.join(HERE, "nvfp4_host", "f32_decisions.c")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), src, "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 mismatches" in r.stdout, r.stdout
