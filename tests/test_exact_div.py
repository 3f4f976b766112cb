"""The quantizers form s_dec_L = amax_B / 6 (NVFP4 paper App. B.2, Eq. 2)
without the fp32 division sequence: fp4exact::div6_normal multiplies by
RN(1/6) and corrects once with the fused remainder.  Its header is plain
C++, compiled here for the host, and checked against fp32 division (the
oracle's arithmetic) on every fp32 input from 2^-125 to FLT_MAX; below
2^-125 (subnormal quotients) the kernels divide, and the check shows why."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "fp4_block_scaled_x16_amd", "csrc")


def test_div6_equals_fp32_division_everywhere_it_is_used(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "div6")
    # fp32 arithmetic as written: no contraction, no fast math; FMA in
    # hardware or libm, correctly rounded either way
    subprocess.run([gxx, "-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-I", CSRC,
                    os.path.join(ROOT, "tests", "div6_exhaustive.cpp"), "-o", exe],
                   check=True, capture_output=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    out = subprocess.run([exe], check=True, capture_output=True, text=True, env=env).stdout
    bad, first, checked, below = (int(v) for v in out.split())
    lo = int(np.float32(2.0 ** -125).view(np.uint32))
    hi = int(np.finfo(np.float32).max.view(np.uint32))
    assert checked == hi - lo + 1
    assert bad == 0, "first mismatch at 0x%08x" % first
    # the fast form does fail on subnormal quotients: the guard is needed
    assert below > 0
