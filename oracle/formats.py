"""Number formats: E2M1 payload, E4M3 / UE5M3 / UE8M0 block scales.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Every encoder here is "nearest value in the table of representable values,
ties to the even code", evaluated with exact float64 distances.  That is the
definition of round-to-nearest-even for a format whose representable values
are listed; it deliberately uses no bit tricks, so it shares no arithmetic
with the device encoders.

Sources
  E2M1 value set {0, .5, 1, 1.5, 2, 3, 4, 6}: NVFP4 pretraining paper, §3
    (background, MXFP4 elements are E2M1: 1 sign, 2 exponent, 1 mantissa bit).
  E4M3 maximum 448 and E2M1 maximum 6: NVFP4 paper, App. B.1 (Eq. 1 prose).
  RNE for the block-scale conversion: NVFP4 paper, App. B.2 (after Eq. 3).
  UE8M0 power-of-two scale 2^-127..2^127: NVFP4 paper, §3.
  UE5M3 (unsigned, 5 exponent bits, 3 mantissa bits): UE5M3 pretraining
    abstract (arXiv 2609.02846).  Bias 15, every code finite, exponent field
    0 read as subnormal: a reading, listed with the others in the design notes.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- E2M1 ----
#: magnitudes of the 8 non-negative E2M1 codes 0..7 (bit 3 is the sign)
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0


def e2m1_value(code):
    """Value of 4-bit E2M1 codes (bit 3 = sign)."""
    code = np.asarray(code).astype(np.int64)
    mag = E2M1_MAG[code & 7]
    return np.where(code & 8, -mag, mag)


def _nearest_code_ties_even(mag, table):
    """Index of the nearest entry of ascending ``table`` to each ``mag``.

    Distances are exact in float64 (both sides have few significant bits and
    neighbours lie within a factor of two).  A tie goes to the even index.
    ``mag`` beyond the last entry maps to the last entry.
    """
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(table, mag, side="left")          # table[hi] >= mag
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_lo = np.abs(mag - table[lo])
    d_hi = np.abs(table[hi] - mag)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


def e2m1_rne(y):
    """E2M1 code of fp32 ``y`` by round-to-nearest-even, saturating at 6.

    Returns (codes uint8 with sign in bit 3, saturated bool array).
    The sign bit copies the sign bit of ``y`` (so -0 gives code 8).
    """
    y = np.asarray(y, dtype=np.float32)
    mag = np.abs(y.astype(np.float64))
    sat = mag > E2M1_MAX
    idx = _nearest_code_ties_even(np.minimum(mag, E2M1_MAX), E2M1_MAG)
    sign = np.signbit(y).astype(np.uint8) << 3
    return (idx.astype(np.uint8) | sign), sat


def e2m1_floor_code(mag):
    """Code of the largest E2M1 magnitude <= ``mag`` (``mag`` in [0, 6])."""
    mag = np.asarray(mag, dtype=np.float64)
    return (np.searchsorted(E2M1_MAG, mag, side="right") - 1).astype(np.int64)


# ------------------------------------------------------- 8-bit scales ----
def _e4m3_table():
    """Values of E4M3 codes 0x00..0x7E (0x7F is NaN and never produced)."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m / 8.0 * 2.0 ** -6)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


def _ue5m3_table():
    """Values of all 256 UE5M3 codes (bias 15, exponent 0 = subnormal)."""
    vals = []
    for code in range(256):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m / 8.0 * 2.0 ** (1 - 15))
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 15))
    return np.array(vals, dtype=np.float64)


E4M3_VALUES = _e4m3_table()
E4M3_MAX = 448.0
UE5M3_VALUES = _ue5m3_table()
UE5M3_MAX = 122880.0

#: number of subnormal (exponent field 0, nonzero) codes: 1..7 in both formats
SUBNORMAL_CODES = range(1, 8)


def _scale_rne_sat(t, table):
    t = np.asarray(t, dtype=np.float32)
    assert np.all(t >= 0) and np.all(np.isfinite(t)), "scale input must be finite, >= 0"
    mag = t.astype(np.float64)
    sat = mag > table[-1]
    idx = _nearest_code_ties_even(np.minimum(mag, table[-1]), table)
    return idx.astype(np.uint8), sat


def _scale_up_sat(t, table):
    """Smallest table value >= t (the code of t rounded up), saturating at
    the largest; `table` is ascending in the code."""
    t = np.asarray(t, dtype=np.float32)
    assert np.all(t >= 0) and np.all(np.isfinite(t)), "scale input must be finite, >= 0"
    mag = t.astype(np.float64)
    sat = mag > table[-1]
    idx = np.searchsorted(table, np.minimum(mag, table[-1]), side="left")
    return idx.astype(np.uint8), sat


def e4m3_up_sat(t):
    """E4M3 code of fp32 ``t >= 0`` rounded up (never below t unless t > 448,
    which saturates to 448)."""
    return _scale_up_sat(t, E4M3_VALUES)


def ue5m3_up_sat(t):
    """UE5M3 code of fp32 ``t >= 0`` rounded up, saturating at 122880."""
    return _scale_up_sat(t, UE5M3_VALUES)


def e4m3_rne_sat(t):
    """E4M3 code of fp32 ``t >= 0``: RNE, saturating at 448 (never NaN).

    Returns (codes uint8, saturated bool array: t > 448).
    """
    return _scale_rne_sat(t, E4M3_VALUES)


def ue5m3_rne_sat(t):
    """UE5M3 code of fp32 ``t >= 0``: RNE, saturating at 122880."""
    return _scale_rne_sat(t, UE5M3_VALUES)


def e4m3_value(code):
    return E4M3_VALUES[np.asarray(code).astype(np.int64)]


def ue5m3_value(code):
    return UE5M3_VALUES[np.asarray(code).astype(np.int64)]


def ue8m0_value(code):
    """2^(code-127) as float64 (code 255, NaN, is never produced)."""
    code = np.asarray(code).astype(np.int64)
    return np.ldexp(1.0, code - 127)


# -------------------------------------------------------- bf16 / fp32 ----
def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x):
    """Round float32 to bf16 (nearest, ties to even); finite inputs only."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)
