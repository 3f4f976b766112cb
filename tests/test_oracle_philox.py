"""Pins for oracle/philox.py.

The oracle's Philox4x32-10 block function is checked against rocRAND's
implementation (public header, compiled here as a host program), which is an
independent library routine for the same published generator.  The 16-bit
stream used by stochastic rounding is then checked for its index mapping and
for uniformity.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox as P

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    subprocess.run([hipcc, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-O1",
                    os.path.join(HERE, "philox_rocrand_ref.cpp"), "-o", exe],
                   check=True, capture_output=True)

    def run(rows):
        inp = "\n".join(" ".join(str(int(v)) for v in r) for r in rows) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return np.array([[int(t) for t in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64)
    return run


def test_block_function_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(123)
    rows = rng.integers(0, 2 ** 32, size=(2000, 6), dtype=np.uint64)
    rows[:4] = [[0, 0, 0, 0, 0, 0], [2 ** 32 - 1] * 6, [1, 0, 0, 0, 1, 0], [0, 0, 1, 0, 7, 0]]
    want = rocrand_ref(rows)
    # the oracle takes a scalar key: evaluate row by row
    got = np.stack([np.array(P.philox4x32_10(*r[:4], r[4], r[5]), dtype=np.uint64) for r in rows])
    assert np.array_equal(got, want)


def test_sr_stream_index_mapping(rocrand_ref):
    seed, offset = (1 << 32) + 5, 3
    idx = np.arange(0, 64, dtype=np.int64)
    r16 = P.sr_random16(idx, seed, offset)
    rows = [[g, 0, offset, 0, seed & 0xFFFFFFFF, seed >> 32] for g in range(8)]
    words = rocrand_ref(rows)
    for i in idx:
        w = int(words[i >> 3][(i & 7) >> 1])
        assert r16[i] == ((w >> (16 * (1 - (i & 1)))) & 0xFFFF)   # even: upper half


def test_sr_stream_uniform_and_seeded():
    idx = np.arange(1 << 20, dtype=np.int64)
    r = P.sr_random16(idx, 1, 0).astype(np.int64)
    counts = np.bincount(r >> 8, minlength=256)
    expected = len(idx) / 256
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)          # ~6 sigma
    assert not np.array_equal(r[:4096], P.sr_random16(idx[:4096], 2, 0))
    assert not np.array_equal(r[:4096], P.sr_random16(idx[:4096], 1, 1))
    # pure function of (index, seed, offset): a shifted window reproduces
    assert np.array_equal(r[1000:3000], P.sr_random16(idx[1000:3000], 1, 0))


def test_rht_sign_mask_is_seeded_input():
    from fp4_block_scaled_x16_amd import inputs
    s = inputs.rht_sign_mask()
    assert 0 <= s < 1 << 16
    assert s == inputs.rht_sign_mask() != inputs.rht_sign_mask(8)
