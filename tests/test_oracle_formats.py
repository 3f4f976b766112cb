"""Pins for oracle/formats.py against the pages and independent routines.

The oracle encodes by "nearest table value, ties to the even code".  These
tests check it against (a) the value set and maxima the NVFP4 paper prints,
(b) textbook round-half-to-even on each binade's grid via numpy.rint, and
(c) torch's float8_e4m3fn and bfloat16 casts (library RNE routines).
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from fp4_block_scaled_x16_amd import inputs
from conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def textbook_round(t, mant_bits, emin, vmax):
    """Round t >= 0 (float64 holding fp32 values) to a binary float format
    with ``mant_bits`` stored mantissa bits, smallest normal exponent
    ``emin`` (subnormals below), saturating at vmax; half to even via rint."""
    t = np.asarray(t, dtype=np.float64)
    _, e = np.frexp(np.maximum(t, 2.0 ** emin))      # t = f 2^e, f in [.5, 1)
    q = np.ldexp(1.0, (e - 1) - mant_bits)            # grid spacing of t's binade
    r = np.rint(t / q) * q
    return np.minimum(r, vmax)


def fp32_probe_values(grid, hi):
    """fp32 values in [0, hi]: a strided sweep of bit patterns plus every
    grid point and midpoint with +-3 ulp neighbours."""
    top = np.float32(hi).view(np.uint32)
    sweep = np.arange(0, int(top), 4099, dtype=np.uint32).view(np.float32)
    pts = np.concatenate([grid, (grid[1:] + grid[:-1]) / 2.0]).astype(np.float32)
    near = [pts]
    up, dn = pts, pts
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        near += [up, dn]
    vals = np.concatenate([sweep] + near + [np.array([hi], np.float32)])
    vals = vals[(vals >= 0) & (vals <= hi)]
    return np.unique(vals)


def test_e2m1_value_set_matches_page():
    g = _golden("e2m1_values.json")
    assert list(F.E2M1_MAG) == g["magnitudes"]
    assert F.E2M1_MAX == g["e2m1_max"]
    assert min(v for v in F.E2M1_MAG if v > 0) == g["e2m1_min_positive"]
    codes = np.arange(16)
    vals = F.e2m1_value(codes)
    assert sorted(set(np.abs(vals).tolist())) == g["magnitudes"]
    assert np.all(vals[8:] == -vals[:8])


def test_e2m1_rne_matches_textbook_rounding():
    vals = fp32_probe_values(F.E2M1_MAG, 16.0)
    codes, sat = F.e2m1_rne(vals)
    got = F.e2m1_value(codes)
    want = textbook_round(vals, 1, 0, 6.0)
    assert np.array_equal(got, want)
    assert np.array_equal(sat, vals.astype(np.float64) > 6.0)
    # negative inputs mirror, including -0 -> code 8
    ncodes, _ = F.e2m1_rne(-vals)
    assert np.array_equal(ncodes, codes | 8)


def test_e2m1_tie_list():
    # the seven exact midpoints go to the code with an even mantissa bit
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])
    codes, _ = F.e2m1_rne(ties)
    assert np.array_equal(F.e2m1_value(codes), want)
    assert np.all(codes % 2 == 0)


def test_e4m3_table_matches_torch():
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(F.E4M3_VALUES, tv)
    assert F.E4M3_VALUES[-1] == _golden("e2m1_values.json")["e4m3_max"]


def test_e4m3_rne_matches_torch_below_max():
    vals = fp32_probe_values(F.E4M3_VALUES, 448.0)
    codes, sat = F.e4m3_rne_sat(vals)
    tc = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, tc)
    assert not sat.any()
    assert np.array_equal(F.e4m3_value(codes), textbook_round(vals, 3, -6, 448.0))


def test_e4m3_saturates_never_nan():
    big = np.array([448.0, 449.0, 463.9, 464.0, 470.0, 1e6, 3.0e38], np.float32)
    codes, sat = F.e4m3_rne_sat(big)
    assert np.all(codes == 0x7E)
    assert sat.tolist() == [False, True, True, True, True, True, True]


def test_ue5m3_structure():
    # exponent field e >= 1 with bias 15 is E4M3's exponent e - 8 with bias 7
    for e in range(1, 16):
        for m in range(8):
            if (e << 3 | m) == 0x7F:
                continue
            assert F.UE5M3_VALUES[((e + 8) << 3) | m] == F.E4M3_VALUES[(e << 3) | m]
    assert F.UE5M3_VALUES[255] == F.UE5M3_MAX == 122880.0
    assert F.UE5M3_VALUES[1] == 2.0 ** -17
    assert np.all(np.diff(F.UE5M3_VALUES) > 0)
    # subnormals continue the grid of exponent field 1
    assert np.allclose(np.diff(F.UE5M3_VALUES[:9]), 2.0 ** -17, rtol=0, atol=0)


def test_ue5m3_rne_matches_textbook_rounding():
    vals = fp32_probe_values(F.UE5M3_VALUES, 2.0 ** 18)
    codes, sat = F.ue5m3_rne_sat(vals)
    assert np.array_equal(F.ue5m3_value(codes), textbook_round(vals, 3, -14, 122880.0))
    assert np.array_equal(sat, vals.astype(np.float64) > 122880.0)


def test_ue8m0_values():
    assert F.ue8m0_value(127) == 1.0
    assert F.ue8m0_value(0) == 2.0 ** -127
    assert F.ue8m0_value(254) == 2.0 ** 127


@pytest.mark.parametrize("fn", [F.f32_to_bf16_bits, inputs.to_bf16_bits])
def test_bf16_rounding_matches_torch(fn):
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-30, 30, 200000)).astype(np.float32)
    # exact ties: bf16 value plus half an ulp
    base = rng.integers(0, 0x7F7F, 50000).astype(np.uint32) << 16   # finite only
    ties = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fn(x), want)
    # and back: exact widening
    assert np.array_equal(F.bf16_bits_to_f32(want),
                          torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())
