"""Exhaustive device checks of the hardware and arithmetic conversions the
hot path relies on, against step functions and values computed from the
oracle's encoders (NVFP4 pretraining paper: §3 for the E2M1 value set and
its maximum 6; App. B.2-B.3 for RNE conversion of block scales and
elements; the UE5M3 abstract for the unsigned E5M3 scale).

* fp32 -> E2M1 RNE: every fp32 pattern except NaNs goes through the packed
  FP4 convert exactly as the quantizer calls it (two values per call into
  byte 0..3 of a word); the expected code is the oracle's rule, evaluated on
  the device as a table of the 7 boundaries between codes, found here by
  bisecting the oracle's encoder over fp32 patterns.
* fp32 -> E2M1 by stochastic rounding (§4.4): every fp32 pattern except
  NaNs through the quantizers' 8-value helper, at an even and an odd
  position, with the 16 random bits just below and at the input's carry
  threshold, against the oracle's rule (round up iff u + floor(65536 f) >=
  65536, f the position between the E2M1 neighbours, which are found by
  bisecting the oracle's round-down code).
* fp32 -> E4M3 / UE5M3 block-scale code: every finite t >= 0 through the
  quantizer's scale encoder, against the 126 / 255 boundaries of the
  oracle's encoders.
* fp32 -> E4M3 MXFP8 element code: every magnitude 0 .. 448 (all that the
  MXFP8 block scale lets through) with both signs at each byte position of
  the hardware FP8 convert's packed word, against the same 126 boundaries
  (the oracle encodes MXFP8 elements with its E4M3 RNE encoder).
* E2M1 x scale -> fp16 (the GEMM operand decode): all 16 codes times every
  E4M3 scale code (the FP4 and FP8 hardware converts, then the packed
  multiply) and every UE5M3 scale code (its packed integer / fp16 decode),
  with the scale in either half of a pair read from either half of a word,
  against the oracle's values rounded to fp16 (exact, checked).
"""
import numpy as np
import pytest

from fp4_block_scaled_x16_amd import api
from oracle import formats as F

pytestmark = pytest.mark.gpu


def _boundaries(encode, n_codes, hi):
    """Smallest fp32 magnitude pattern whose code is k, for k = 1 .. n_codes-1,
    by bisection of a monotone encoder over patterns [0, hi]."""
    lo_b = np.zeros(n_codes - 1, np.int64)            # code(lo_b) < k
    hi_b = np.full(n_codes - 1, hi, np.int64)          # code(hi_b) >= k
    k = np.arange(1, n_codes)
    assert np.all(encode(np.array([0], np.uint32))[0] == 0)
    assert np.all(encode(np.full(1, hi, np.uint32))[0] == n_codes - 1)
    while np.any(hi_b - lo_b > 1):
        mid = (lo_b + hi_b) // 2
        up = encode(mid.astype(np.uint32)) >= k
        hi_b = np.where(up, mid, hi_b)
        lo_b = np.where(up, lo_b, mid)
    return hi_b.astype(np.uint32)


def _as_f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def test_e2m1_rne_convert_exhaustive():
    thr = _boundaries(lambda b: F.e2m1_rne(_as_f32(b))[0].astype(np.int64) & 7, 8, 0x7F800000)
    # the boundaries are the midpoints of the value set, a tie going to the
    # even code (reading of App. B.3: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1,
    # 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4)
    nxt = lambda v: np.nextafter(np.float32(v), np.float32(np.inf))
    want = np.array([nxt(0.25), 0.75, nxt(1.25), 1.75, nxt(2.5), 3.5, nxt(5.0)], np.float32)
    assert np.array_equal(_as_f32(thr), want)
    bad, first, checked = api.selftest_sweep("e2m1_rne", thr)
    assert checked == 2 ** 32 - (2 ** 24 - 2)
    assert bad == 0, "%d mismatches, first at 0x%08x" % (bad, first)


def test_e2m1_sr_exhaustive():
    # the round-down code steps at the E2M1 magnitudes themselves (§3)
    thr = _boundaries(lambda b: F.e2m1_floor_code(np.abs(_as_f32(b))), 8, 0x7F800000)
    assert np.array_equal(_as_f32(thr), np.array([0.5, 1, 1.5, 2, 3, 4, 6], np.float32))
    # every input, at an even and an odd element position, with the random
    # value just below and at its carry threshold (the rule of the oracle's
    # stochastic rounding: u + floor(65536 f) >= 65536)
    bad, first, checked = api.selftest_sweep("e2m1_sr", thr)
    assert checked == 4 * (2 ** 32 - (2 ** 24 - 2))
    assert bad == 0, "%d mismatches, first at 0x%08x" % (bad, first)


@pytest.mark.parametrize("kind,encode,n_codes,vmax", [
    ("e4m3_scale", F.e4m3_rne_sat, 0x7F, F.E4M3_MAX),
    ("ue5m3_scale", F.ue5m3_rne_sat, 256, F.UE5M3_MAX),
])
def test_scale_encoder_exhaustive(kind, encode, n_codes, vmax):
    thr = _boundaries(lambda b: encode(_as_f32(b))[0].astype(np.int64), n_codes, 0x7F7FFFFF)
    assert len(thr) == n_codes - 1
    # the top boundary lies between the two largest values (saturation
    # above the maximum is the rest of the last step)
    assert _as_f32(thr[-1]) <= vmax
    bad, first, checked = api.selftest_sweep(kind, thr)
    assert checked == 0x7F800000
    assert bad == 0, "%d mismatches, first at 0x%08x" % (bad, first)


def test_mxfp8_element_encoder_exhaustive():
    thr = _boundaries(lambda b: F.e4m3_rne_sat(_as_f32(b))[0].astype(np.int64), 0x7F, 0x7F7FFFFF)
    # code k begins at the midpoint between values k-1 and k, a tie going
    # to the even code: at the midpoint for even k, just above it for odd k
    vals = F.E4M3_VALUES[:0x7F].astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)      # exact: 4 mantissa bits
    k = np.arange(1, 0x7F)
    want = np.where(k % 2 == 0, mids, np.nextafter(mids, np.float32(np.inf)))
    assert np.array_equal(_as_f32(thr), want)
    bad, first, checked = api.selftest_sweep("e4m3_elem", thr)
    assert checked == 0x43E00001                      # every pattern 0 .. 448.0f
    assert bad == 0, "%d mismatches, first at 0x%08x" % (bad, first)


@pytest.mark.parametrize("fmt,values,shift,n_codes", [
    ("nvfp4", F.E4M3_VALUES, 1.0, 0x7F),
    ("ue5m3", F.UE5M3_VALUES, 2.0 ** -5, 256),
])
def test_gemm_operand_decode_exhaustive(fmt, values, shift, n_codes):
    got = api.selftest_gemm_decode(fmt)                      # [256, 4, 16]
    e2m1 = F.e2m1_value(np.arange(16))                        # codes 0..15
    exact = values[:n_codes, None] * e2m1[None, :] * shift    # float64
    half = exact.astype(np.float16)
    assert np.array_equal(half.astype(np.float64), exact)     # premise: exact in fp16
    want = half.view(np.uint16)                               # code 8 gives -0
    assert want[1, 8] == 0x8000
    for v in range(4):      # scale in either half of a pair from bytes 0-1 or 2-3
        assert np.array_equal(got[:n_codes, v], want), (fmt, v, np.argwhere(got[:n_codes, v] != want)[:5])
    assert not got[n_codes:].any()
