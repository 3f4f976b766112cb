"""Pins for oracle/quantize.py against what the pages fix.

  * a hand-derived NVFP4 example (App. B.1-B.3 with exact powers of two)
  * the MXFP4 worked example of App. B.4 (amax = 3 + eps)
  * block amax maps to the FP4 maximum 6 (§3, App. B.2) for RNE blocks with
    a normal scale, and is recovered to within E4M3 precision (§3: the block
    amax is kept at near-FP8 precision)
  * idempotence: quantize(dequantize(q)) == q
  * 2D scaling is transposition invariant (§4.3; 2D-block FP4 abstract)
  * stochastic rounding is unbiased (§4.4) and never moves on-grid values
  * event counters on crafted blocks whose counts follow from the rules
"""
import json
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import quantize as Q
from oracle.rht import rht16_cols
from fp4_block_scaled_x16_amd import inputs
from conftest import GOLDEN


def bits(a):
    return inputs.to_bf16_bits(np.asarray(a, np.float32))


def test_hand_example_nvfp4():
    # Block 0 has amax 6, block 1 has amax 10.5 = the tensor amax.
    # Eq. 1: s_enc = 2688 / 10.5 = 256 exactly, s_dec = 2^-8.
    # Block 0: Eq. 2 s_dec_L = 1, Eq. 3 t = 256 -> E4M3 256 (code 0x78),
    # s_enc_L = 1 / (256 * 2^-8) = 1, so y = x and codes are plain RNE of x.
    b0 = [6, -0.5, 1, 1.5, 2, 3, 4, -6, 0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5]
    want0 = [7, 9, 2, 3, 4, 5, 6, 15, 0, 0, 2, 2, 4, 4, 6, 6]
    # Block 1: t = 10.5 / 6 * 256 = 448 -> code 0x7E; s_enc_L = fp32(1 / 1.75)
    # which rounds up (4/7 = 0.100100...b), so y(10.5) = 6 + tiny > 6:
    # saturated, code 7.  Other entries: 1.75 * 4/7 = 1 -> code 2.
    b1 = [10.5] + [1.75] * 15
    q = Q.quantize(bits([b0 + b1]), "nvfp4")
    assert q["amax"] == np.float32(10.5)
    assert q["s_dec"] == np.float32(2.0 ** -8)
    assert q["scales"].tolist() == [[0x78, 0x7E]]
    assert q["codes_unpacked"][0, :16].tolist() == want0
    assert q["codes_unpacked"][0, 16:].tolist() == [7] + [2] * 15
    # packing: even element in the low nibble
    assert q["codes"][0, 0] == (want0[0] | want0[1] << 4)
    c = q["counters"]
    assert c["elem_saturated"] == 1
    assert c["elem_underflow"] == 1          # 0.25 -> 0; the exact 0 is not an event
    assert c["scale_saturated"] == c["scale_underflow"] == c["scale_subnormal"] == 0


def test_mxfp4_worked_example():
    with open(os.path.join(GOLDEN, "mxfp4_amax_3_plus_eps.json")) as f:
        g = json.load(f)
    rng = np.random.default_rng(1)
    eps = np.float32(2.0 ** -6)
    blk = rng.uniform(-3, 3, 32).astype(np.float32)
    blk[5] = 3 + eps
    q = Q.quantize(bits([blk]), "mxfp4")
    assert q["scales"].tolist() == [[g["ue8m0_code"]]]
    assert F.ue8m0_value(q["scales"][0, 0]) == g["decode_scale"]
    mags = q["codes_unpacked"][0] & 7
    assert mags[5] == g["amax_element_code_magnitude"]
    assert F.E2M1_MAG[mags[5]] == g["amax_element_value"]
    used = set(F.E2M1_MAG[mags].tolist())
    assert not used & set(g["unused_magnitudes"])
    assert np.isclose(np.log2(3 / 0.5), g["binades_used"])
    assert np.isclose(np.log2(6 / 0.5), g["binades_full"])


def test_mx_scale_is_smallest_nonsaturating_power_of_two():
    rng = np.random.default_rng(2)
    a = (rng.uniform(0.5, 1, 5000) * 2.0 ** rng.integers(-120, 120, 5000)).astype(np.float32)
    a = np.concatenate([a, np.float32(6.0) * np.float32(2.0) ** np.arange(-20, 20, dtype=np.float32)])
    code, s_enc, _ = Q.block_scales_mx(a)
    e = code.astype(np.int64) - 127
    for ai, ei in zip(a.tolist(), e.tolist()):
        from fractions import Fraction
        A = Fraction(ai)
        assert 6 * Fraction(2) ** ei >= A > 6 * Fraction(2) ** (ei - 1)
    assert np.array_equal(s_enc, np.ldexp(1.0, -e).astype(np.float32))


def _blocks_with_normal_scale(q, fmt, bs):
    codes = q["codes_unpacked"]
    R, C = codes.shape
    sc = q["scales"].reshape(R, C // bs)
    return codes.reshape(R, C // bs, bs), sc, sc >= 8


@pytest.mark.parametrize("fmt,target", [("nvfp4", 448.0), ("ue5m3", 448.0), ("ue5m3", 2048.0)])
def test_block_amax_maps_to_six(fmt, target):
    x = inputs.activations((64, 1024), cfg_seed=3)
    dy = inputs.gradients((64, 1024), cfg_seed=3)
    for t in (x, dy):
        q = Q.quantize(t, fmt, target=target)
        cb, sc, normal = _blocks_with_normal_scale(q, fmt, 16)
        xf = F.bf16_bits_to_f32(t).reshape(cb.shape)
        arg = np.abs(xf).argmax(axis=2)
        amax_code = np.take_along_axis(cb, arg[..., None], axis=2)[..., 0] & 7
        assert normal.sum() > 0.9 * normal.size
        assert np.all(amax_code[normal] == 7)


def test_block_amax_near_fp8_precision():
    x = inputs.activations((64, 2048), cfg_seed=4)
    q = Q.quantize(x, "nvfp4")
    cb, sc, normal = _blocks_with_normal_scale(q, "nvfp4", 16)
    xf = F.bf16_bits_to_f32(x).reshape(cb.shape).astype(np.float64)
    amax_b = np.abs(xf).max(axis=2)
    dq_amax = 6.0 * F.e4m3_value(sc) * np.float64(q["s_dec"])
    ok = normal & (sc < 0x7E)
    rel = np.abs(dq_amax - amax_b) / amax_b
    assert np.all(rel[ok] <= 2.0 ** -4 * (1 + 1e-6))


@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3", "mxfp4"])
def test_idempotent(fmt):
    # q(dq(q(x))) == q(x) on every block whose largest code is the format
    # maximum; dequantized values are rounded to bf16 (the quantizer input)
    x = inputs.activations((32, 1024), cfg_seed=5)
    R, C = x.shape
    bs = Q.BLOCK[fmt]
    q1 = Q.quantize(x, fmt)
    dq = Q.dequantize(q1["codes"], q1["scales"], fmt, "1d", q1["s_dec"], R, C, out="bf16")
    q2 = Q.quantize(dq, fmt)
    c1 = q1["codes_unpacked"].reshape(R, C // bs, bs)
    c2 = q2["codes_unpacked"].reshape(R, C // bs, bs)
    maxmag = (c1 & 7).max(axis=2)
    full = maxmag >= (6 if fmt == "mxfp4" else 7)
    if fmt != "mxfp4":
        full &= q1["scales"] >= 8
    assert full.mean() > (0.75 if fmt == "mxfp4" else 0.9)
    assert np.array_equal(c1[full], c2[full])
    assert np.array_equal(q1["scales"][full], q2["scales"][full])
    if fmt != "mxfp4":
        # s_dec passed through (the amax given) also reproduces the codes
        q3 = Q.quantize(dq, fmt, amax=q1["amax"])
        c3 = q3["codes_unpacked"].reshape(R, C // bs, bs)
        assert np.array_equal(c1[full], c3[full])


def test_mx_max_code_three_is_value_preserving():
    # App. B.4 case: requantizing halves the scale and doubles the codes
    blk = np.zeros((1, 32), np.float32)
    blk[0, :4] = [3.125, 1.0, -0.5, 2.0]
    q1 = Q.quantize(bits(blk), "mxfp4")
    dq = Q.dequantize(q1["codes"], q1["scales"], "mxfp4", "1d", 1.0, 1, 32)
    q2 = Q.quantize(bits(dq), "mxfp4")
    dq2 = Q.dequantize(q2["codes"], q2["scales"], "mxfp4", "1d", 1.0, 1, 32)
    assert np.array_equal(dq, dq2)
    assert q2["scales"][0, 0] == q1["scales"][0, 0] - 1


@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3"])
def test_2d_transposition_invariant(fmt):
    w = inputs.weights((96, 160), cfg_seed=6)
    q = Q.quantize(w, fmt, block="2d", emit_transpose=True)
    qt = Q.quantize(np.ascontiguousarray(w.T), fmt, block="2d", emit_transpose=True)
    assert np.array_equal(q["codes_unpacked"].T, qt["codes_unpacked"])
    assert np.array_equal(q["scales"].T, qt["scales"])
    assert np.array_equal(q["codes_t"], qt["codes"])
    assert np.array_equal(qt["codes_t"], q["codes"])
    assert q["scales"].shape == (6, 10)


def test_colwise_is_rowwise_of_transpose():
    x = inputs.gradients((64, 96), cfg_seed=7)
    for rnd in ("rne", "sr"):
        a = Q.quantize(x, "nvfp4", orient="col", rnd=rnd, seed=1, offset=1)
        b = Q.quantize(np.ascontiguousarray(x.T), "nvfp4", orient="row", rnd=rnd, seed=1, offset=1)
        for k in ("codes", "scales", "amax", "s_dec"):
            assert np.array_equal(a[k], b[k])
        assert a["counters"] == b["counters"]


def test_rht_amax_after_rotation():
    x = inputs.activations((64, 48), cfg_seed=8)
    s = inputs.rht_sign_mask()
    q = Q.quantize(x, "nvfp4", orient="col", rht=True, signs=s)
    rot = rht16_cols(F.bf16_bits_to_f32(x), s)
    assert q["amax"] == np.float32(np.abs(rot).max())
    assert q["amax"] != np.float32(np.abs(F.bf16_bits_to_f32(x)).max())


def _sr_codes_and_y(x_bits, reps, seed=1):
    """Codes for reps SR repetitions (offset = repetition) and y = x * s_enc_L."""
    xf = F.bf16_bits_to_f32(x_bits)
    R, C = xf.shape
    amax = Q.tensor_amax(xf)
    s_enc, s_dec = Q.global_scales(amax)
    amax_b = np.abs(xf.reshape(R, C // 16, 16)).max(axis=2)
    _, s_enc_l, _ = Q.block_scales_two_level(amax_b, s_enc, s_dec, "nvfp4")
    y = (xf * np.repeat(s_enc_l, 16, axis=1)).astype(np.float32).astype(np.float64)
    codes = [Q.quantize(x_bits, "nvfp4", rnd="sr", seed=seed, offset=r)["codes_unpacked"]
             for r in range(reps)]
    return np.stack(codes), y


def test_sr_unbiased_config1():
    # Tiny workload: A = 256 x 256 ~ N(0, 1), seed 0; SR with Philox seed 1,
    # 100 repetitions -> 6.5M draws.  Over unclipped elements the mean of
    # (value(code) - y) must be within 3 standard errors of 0.
    a = inputs.linear_tensors(1)["X"]
    codes, y = _sr_codes_and_y(a, 100)
    vals = F.e2m1_value(codes)                        # [reps, R, C]
    keep = np.abs(y) <= 6.0
    err = (vals - y[None])[:, keep].ravel()
    n = err.size
    assert n >= 10 ** 6
    se = err.std() / np.sqrt(n)
    assert abs(err.mean()) < 3 * se
    # RNE on the same data is biased well beyond that (sanity of the test)
    rne = F.e2m1_value(Q.quantize(a, "nvfp4")["codes_unpacked"])
    assert abs((rne - y)[keep].mean()) > 3 * se


def test_sr_matches_exact_expectation_and_keeps_grid_values():
    a = inputs.linear_tensors(1)["X"][:64]
    codes, y = _sr_codes_and_y(a, 40)
    m = np.abs(y)
    vals = np.abs(F.e2m1_value(codes))
    keep = m <= 6
    # neighbours on the E2M1 value set (NVFP4 paper §3), found here by
    # search rather than with the oracle's own encoder
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    k = np.minimum(np.searchsorted(grid, np.minimum(m, 6.0), side="right") - 1, 6)
    lo, hi = grid[k], grid[k + 1]
    # every draw lands on one of the two neighbours
    assert np.all((vals[:, keep] == lo[keep]) | (vals[:, keep] == hi[keep]) | (m[keep] == 6))
    # aggregate of (empirical mean - exact expectation) is ~ N(0, se)
    frac = (m - lo) / (hi - lo)
    p_up = np.floor(frac * 65536) / 65536
    expect = lo + (hi - lo) * p_up
    var = (hi - lo) ** 2 * p_up * (1 - p_up)
    d = (vals[:, keep].mean(axis=0) - expect[keep])
    z = d.sum() / np.sqrt((var[keep] / codes.shape[0]).sum())
    assert abs(z) < 4


def test_sr_rule_over_every_random_value():
    # One element against all 65536 values of its 16 random bits: the draws
    # that round up must be exactly the r with r + floor(65536 f) >= 65536,
    # f the position of |y| between its E2M1 neighbours (found by search on
    # the value set, NVFP4 paper §3), so that P(up) = floor(65536 f) / 65536;
    # when 65536 f is an integer the mean over all r is |y| exactly (§4.4:
    # unbiased).  Cases: each interval of the value set, fractions on and
    # just off a multiple of 2^-16, tiny fractions, the top of [4, 6), 6 and
    # beyond, and negative values.
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    ys = []
    for lo, hi in zip(grid[:-1], grid[1:]):
        for f in (0.0, 0.5, 0.25, 0.2, 1 / 3, 12345 / 65536, (12345 + 2 ** -6) / 65536,
                  (12345 - 2 ** -6) / 65536, 2 ** -17, 2 ** -20, 1 - 2 ** -16, 1 - 2 ** -20):
            ys.append(np.float32(lo + f * (hi - lo)))
    ys += [np.float32(6.0), np.float32(7.5), np.float32(1e30)]
    ys += [-y for y in ys[:40]]
    r = np.arange(65536, dtype=np.uint16)
    for y in ys:
        v = np.full(65536, y, np.float32)
        codes, _, _ = Q.encode_elements(v, np.float32(1.0), "sr", r)
        assert np.all((codes >> 3) == (1 if np.signbit(y) else 0))
        vals = np.abs(F.e2m1_value(codes))
        m = abs(float(y))
        if m >= 6:
            assert np.all(vals == 6.0)
            continue
        k = np.searchsorted(grid, m, side="right") - 1
        lo, hi = grid[k], grid[k + 1]
        lead = int(np.floor((m - lo) / (hi - lo) * 65536))
        up = vals == hi
        assert np.all(up | (vals == lo))
        assert np.array_equal(up, r.astype(np.int64) >= 65536 - lead), y
        if ((m - lo) / (hi - lo) * 65536).is_integer():
            assert vals.mean() == m


def test_sr_keeps_on_grid_values():
    # s_enc = 256, s_dec = 2^-8 and block scale 256 give s_enc_L = 1, so
    # y = x: on-grid values (including 0) must never be moved by SR
    grid = [6, 4, 3, 2, 1.5, 1, 0.5, 0, -0.5, -1, -1.5, -2, -3, -4, -6, 0]
    x = bits([grid + [10.5] + [0.0] * 15])
    for r in range(200):
        q = Q.quantize(x, "nvfp4", rnd="sr", seed=1, offset=r)
        assert np.array_equal(F.e2m1_value(q["codes_unpacked"][0, :16]), np.array(grid, float))


def test_sr_reproducible():
    dy = inputs.gradients((32, 256), cfg_seed=9)
    a = Q.quantize(dy, "nvfp4", rnd="sr", seed=1, offset=0)
    b = Q.quantize(dy, "nvfp4", rnd="sr", seed=1, offset=0)
    c = Q.quantize(dy, "nvfp4", rnd="sr", seed=1, offset=1)
    assert np.array_equal(a["codes"], b["codes"])
    assert not np.array_equal(a["codes"], c["codes"])


def test_counters_outlier_underflow():
    # one 1e30 element: s_enc = 2688 / 1e30, so a block with amax ~1e-10 has
    # t ~ 4e-38 -> E4M3 code 0: every other nonzero block underflows, and all
    # its nonzero elements become +-0.
    x = np.full((4, 64), 1e-10, np.float32)
    x[1, 3] = 1e30
    x[2, 16:32] = 0.0
    q = Q.quantize(bits(x), "nvfp4")
    c = q["counters"]
    nonzero_blocks = 16 - 1 - 1
    assert c["scale_underflow"] == nonzero_blocks
    assert c["elem_underflow"] == nonzero_blocks * 16 + 15
    assert c["scale_saturated"] == 0
    assert np.all(q["codes_unpacked"][0] == 0)


def test_counters_zero_tensor_and_signed_zero():
    x = np.zeros((2, 32), np.float32)
    x[1, 5] = -0.0
    q = Q.quantize(bits(x), "nvfp4")
    assert q["amax"] == 0 and q["s_dec"] == 1.0
    assert np.all(q["scales"] == 0)
    assert q["codes_unpacked"][1, 5] == 8 and q["codes_unpacked"][0, 5] == 0
    assert q["counters"] == Q.zero_counters()


def test_counters_stale_amax_saturation():
    # With a stale amax a_s, block scale t = amax_B / a_s * T saturates
    # E4M3 exactly when amax_B / a_s * 448 > 448 (up to fp32 rounding).
    x = inputs.activations((64, 512), cfg_seed=10)
    xf = F.bf16_bits_to_f32(x)
    amax_b = np.abs(xf.reshape(64, 32, 16)).max(axis=2).astype(np.float64)
    a_s = np.float32(np.abs(xf).max() / 8.0)
    q = Q.quantize(x, "nvfp4", amax=a_s)
    ratio = amax_b / np.float64(a_s)
    clear_sat = (ratio > 1 + 1e-6).sum()
    clear_ok = (ratio < 1 - 1e-6).sum()
    assert clear_sat <= q["counters"]["scale_saturated"] <= amax_b.size - clear_ok
    # the same data under UE5M3 (max 122880) does not saturate its scales
    q5 = Q.quantize(x, "ue5m3", amax=a_s, target=2048.0)
    assert q5["counters"]["scale_saturated"] == 0
    # with E4M3 saturated at 448, y = x * 6 / a_s: every |x| > a_s clips
    n_big = int((np.abs(xf) > a_s * (1 + 1e-6)).sum())
    assert n_big > 0 and q["counters"]["elem_saturated"] >= n_big


def test_ue5m3_larger_target_avoids_scale_underflow():
    # t = T * amax_B / amax.  With amax = 1 and a block of amax 2^-27:
    # T = 448 gives t = 0.875 * 2^-18, below half the smallest UE5M3 value
    # (2^-17), so the scale underflows to 0; T = 2048 gives t = 2^-16, a
    # subnormal scale (code 2).  (UE5M3 abstract: larger T, fewer underflows.)
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    x[0, 16:] = 2.0 ** -27
    a = Q.quantize(bits(x), "ue5m3", target=448.0)
    b = Q.quantize(bits(x), "ue5m3", target=2048.0)
    assert a["scales"][0, 1] == 0 and a["counters"]["scale_underflow"] == 1
    assert a["counters"]["elem_underflow"] == 16
    assert b["scales"][0, 1] == 2 and b["counters"]["scale_underflow"] == 0
    assert b["counters"]["scale_subnormal"] == 1


def test_format_error_ordering_small_band():
    # §3: NVFP4 (16-blocks, E4M3 scales) is more accurate than MXFP4
    x = inputs.activations((64, 1024), cfg_seed=12)
    xf = F.bf16_bits_to_f32(x).astype(np.float64)
    errs = {}
    for fmt in ("nvfp4", "mxfp4"):
        q = Q.quantize(x, fmt)
        dq = Q.dequantize(q["codes"], q["scales"], fmt, "1d", q["s_dec"] if q["s_dec"] else 1.0, 64, 1024)
        errs[fmt] = np.linalg.norm(dq - xf) / np.linalg.norm(xf)
    assert errs["nvfp4"] < errs["mxfp4"]
    assert 0.05 < errs["nvfp4"] < 0.2


def test_dequantize_bf16_is_rounded_f32():
    import torch
    dy = inputs.gradients((16, 256), cfg_seed=13)
    q = Q.quantize(dy, "ue5m3", rnd="sr", seed=1)
    f = Q.dequantize(q["codes"], q["scales"], "ue5m3", "1d", q["s_dec"], 16, 256)
    b = Q.dequantize(q["codes"], q["scales"], "ue5m3", "1d", q["s_dec"], 16, 256, out="bf16")
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, want)


def test_empty_tensor():
    x = np.zeros((0, 32), np.uint16)
    q = Q.quantize(x, "nvfp4")
    assert q["codes"].shape == (0, 16) and q["scales"].shape == (0, 2)
    assert q["amax"] == 0 and q["s_dec"] == 1


# --------------------------------- truncation-free scales and 2D SR --------
# (2D-block FP4 page: 2D blocks combined with truncation-free scaling and
# stochastic rounding keep gradients unbiased)


@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3"])
def test_round_up_scale_is_smallest_value_not_below(fmt):
    table = F.E4M3_VALUES if fmt == "nvfp4" else F.UE5M3_VALUES
    enc = F.e4m3_up_sat if fmt == "nvfp4" else F.ue5m3_up_sat
    rng = np.random.default_rng(21)
    t = np.concatenate([table.astype(np.float32),                       # exactly representable
                        (rng.uniform(0, 1, 20000) * table[-1]).astype(np.float32),
                        np.float32(2.0) ** rng.uniform(-24, 10, 20000).astype(np.float32)])
    t = t[t <= table[-1]]
    code, sat = enc(t)
    assert not sat.any()
    v = table[code]
    assert np.all(v >= t.astype(np.float64))                  # never below
    below = code > 0
    assert np.all(table[code[below] - 1] < t[below])           # and the smallest such
    # on representable inputs it agrees with round-to-nearest
    exact = np.isin(t.astype(np.float64), table)
    rne = (F.e4m3_rne_sat if fmt == "nvfp4" else F.ue5m3_rne_sat)(t[exact])[0]
    assert np.array_equal(code[exact], rne)
    c, s = enc(np.float32([table[-1] * 2]))
    assert c[0] == len(table) - 1 and s[0]


@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3"])
@pytest.mark.parametrize("block", ["1d", "2d"])
def test_round_up_scales_leave_nothing_to_clip(fmt, block):
    x = inputs.activations((256, 256), cfg_seed=3)          # N(0,1) with x50 outliers
    up = Q.quantize(x, fmt, block=block, scale_round="up")
    rne = Q.quantize(x, fmt, block=block)
    assert rne["counters"]["elem_saturated"] > 0            # nearest scales do clip
    assert up["counters"]["elem_saturated"] == 0            # rounded-up ones do not
    # the scale codes are the nearest ones or one above
    d = up["scales"].astype(int) - rne["scales"].astype(int)
    assert set(np.unique(d)) <= {0, 1}


def test_2d_sr_is_transposition_consistent_and_unbiased():
    w = inputs.weights((64, 48), cfg_seed=4)
    q = Q.quantize(w, "nvfp4", block="2d", rnd="sr", seed=9, offset=0, emit_transpose=True,
                   scale_round="up")
    codes = Q.unpack_codes(q["codes"])
    assert np.array_equal(Q.unpack_codes(q["codes_t"]), codes.T)
    # transposing W and quantizing again gives the transposed result only with
    # the same random bits; with the bits of W^T's own layout it differs
    qt = Q.quantize(np.ascontiguousarray(w.T), "nvfp4", block="2d", rnd="sr", seed=9, offset=0,
                    scale_round="up")
    assert np.array_equal(qt["scales"], q["scales"].T)
    # unbiased over 200 draws: no element is clipped, so every element's mean
    # code value converges to y (3 sigma on the pooled mean)
    xf = F.bf16_bits_to_f32(w).astype(np.float64)
    vals = []
    for r in range(200):
        qr = Q.quantize(w, "nvfp4", block="2d", rnd="sr", seed=9, offset=r, scale_round="up")
        vals.append(Q.operand_values(qr["codes"], qr["scales"], "nvfp4", "2d", 64, 48)
                    * float(qr["s_dec"]))
    err = np.stack(vals) - xf[None]
    scale = Q.element_scales(q["scales"], "nvfp4", "2d", 64, 48) * float(q["s_dec"])
    z = err / scale[None]                                   # in units of the element's scale
    assert q["counters"]["elem_saturated"] == 0
    assert abs(z.mean()) < 3 * z.std() / np.sqrt(z.size)


def test_format_error_ordering():
    """NVFP4 paper §3 (App. B.4 worked example): 16-element blocks with
    E4M3 scales represent values more accurately than 32-element blocks
    with power-of-two scales.  On rows drawn like the format-comparison
    workload's X, W and dY (1D blocks, SR on dY), NVFP4's relative
    Frobenius quantization error is below MXFP4's for every tensor."""
    shapes = {"X": (128, 4096), "W": (128, 4096), "dY": (64, 21504)}
    gens = {"X": inputs.activations, "W": inputs.weights, "dY": inputs.gradients}
    for name, shape in shapes.items():
        x = gens[name](shape, cfg_seed=0)
        xf = F.bf16_bits_to_f32(x).astype(np.float64)
        kw = dict(rnd="sr", seed=1) if name == "dY" else {}
        err = {}
        for fmt in ("nvfp4", "mxfp4"):
            q = Q.quantize(x, fmt, **kw)
            dq = Q.dequantize(q["codes"], q["scales"], fmt, "1d", q["s_dec"], *shape)
            err[fmt] = np.linalg.norm(dq.astype(np.float64) - xf) / np.linalg.norm(xf)
        assert err["nvfp4"] < err["mxfp4"], (name, err)


# ------------------------- RHT on the Fprop / Dgrad operands (along K) ----
@pytest.mark.parametrize("n", [4, 16, 32, 64, 128])
@pytest.mark.parametrize("fmt,rnd", [("nvfp4", "rne"), ("ue5m3", "sr")])
def test_rowwise_rht_is_colwise_rht_of_transpose(n, fmt, rnd):
    """NVFP4 paper §4.2 (RHT on Fprop / Dgrad inputs): rotating along the
    rows of X (rowwise blocks) is the pinned column rotation of X^T: the
    rowwise quantization of X with the RHT equals, code for code, the
    colwise quantization of X^T with the same transform and signs (SR
    indices are those of the same output code matrix)."""
    x = inputs.activations((48, 2 * n if n >= 64 else 128), cfg_seed=60 + n)
    s = inputs.rht_sign_bits(n)
    a = Q.quantize(x, fmt, orient="row", rnd=rnd, seed=3, offset=1, rht=True, signs=s, rht_n=n)
    b = Q.quantize(np.ascontiguousarray(x.T), fmt, orient="col", rnd=rnd, seed=3, offset=1,
                   rht=True, signs=s, rht_n=n)
    for k in ("codes", "scales", "amax", "s_dec"):
        assert np.array_equal(a[k], b[k]), k
    assert a["counters"] == b["counters"]


def test_fprop_with_rotated_operands_approximates_the_product():
    """Fprop with X and W rotated along K by the same D_r H16 (§4.2): the
    rotation cancels in X W^T (H orthonormal), so the product of the
    dequantized rotated operands approximates X W^T as closely as the
    unrotated quantized product does: relative Frobenius error below 0.2 for
    both (each operand carries an E2M1 relative RMS error near 0.085, so the
    product's is near 0.12; a rotation that does not cancel gives an error
    near 1), within a factor 1.5 of each other."""
    X = inputs.activations((256, 512), cfg_seed=61)
    W = inputs.weights((128, 512), cfg_seed=61)
    ref = F.bf16_bits_to_f32(X).astype(np.float64) @ F.bf16_bits_to_f32(W).astype(np.float64).T
    s = inputs.rht_sign_mask()
    errs = []
    for rht in (False, True):
        qx = Q.quantize(X, "nvfp4", rht=rht, signs=s)
        qw = Q.quantize(W, "nvfp4", rht=rht, signs=s)
        dx = Q.dequantize(qx["codes"], qx["scales"], "nvfp4", "1d", qx["s_dec"], 256, 512)
        dw = Q.dequantize(qw["codes"], qw["scales"], "nvfp4", "1d", qw["s_dec"], 128, 512)
        d = dx.astype(np.float64) @ dw.astype(np.float64).T
        errs.append(np.linalg.norm(d - ref) / np.linalg.norm(ref))
    assert max(errs) < 0.2 and errs[1] < 1.5 * errs[0] and errs[0] < 1.5 * errs[1], errs


# ---------------------------------------------- per-row global scale ----
# NVFP4 paper App. B.1, last sentence: the global scale may span a row
# instead of the whole tensor, so no separate amax pass is needed.

def _rows_over_decades(R, C, cfg_seed):
    """bf16 bits of an [R, C] matrix whose rows differ in scale by up to
    2^40 (row r is N(0, 1) times 2^(2 (r mod 21) - 20))."""
    v = inputs.normal((R, C), cfg_seed=cfg_seed)
    f = np.exp2(2.0 * (np.arange(R) % 21) - 20.0).astype(np.float32)
    return bits(F.bf16_bits_to_f32(v) * f[:, None])


@pytest.mark.parametrize("fmt,target", [("nvfp4", 448.0), ("ue5m3", 2048.0)])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_row_scope_quantizes_each_row_as_a_one_row_tensor(fmt, target, rnd):
    """With the global scale spanning a row, row r is quantized exactly as
    the 1 x C tensor x[r] with its own tensor amax (the row amax); under SR
    the row keeps its random bits (index r * C + c, passed as index_base)."""
    R, C = 24, 64
    x = _rows_over_decades(R, C, 11)
    q = Q.quantize(x, fmt, rnd=rnd, seed=5, offset=2, target=target, scope="row")
    total = Q.zero_counters()
    for r in range(R):
        q1 = Q.quantize(x[r:r + 1], fmt, rnd=rnd, seed=5, offset=2, target=target,
                        index_base=r * C)
        assert np.array_equal(q["codes"][r], q1["codes"][0])
        assert np.array_equal(q["scales"][r], q1["scales"][0])
        assert q["amax"][r] == q1["amax"] and q["s_dec"][r] == q1["s_dec"]
        for k in total:
            total[k] += q1["counters"][k]
    assert q["counters"] == total
    assert q["s_dec"].dtype == np.float32 and q["s_dec"].shape == (R,)


@pytest.mark.parametrize("fmt,target,rne_sat", [("nvfp4", 448.0, F.e4m3_rne_sat),
                                                 ("ue5m3", 2048.0, F.ue5m3_rne_sat)])
def test_row_scope_every_row_reaches_the_target_scale(fmt, target, rne_sat):
    """Eq. 1 per row maps each row's largest local decode scale amax_r / 6
    to T, so every nonzero row holds a block whose scale code is the code of
    T (448: E4M3 0x7E; 2048: UE5M3 2^11).  With one tensor scale only the
    row holding the tensor amax does."""
    x = _rows_over_decades(42, 64, 12)
    want = int(rne_sat(np.array([target], np.float32))[0][0])
    q = Q.quantize(x, fmt, target=target, scope="row")
    assert np.all(q["scales"].max(axis=1) == want)
    qt = Q.quantize(x, fmt, target=target)
    assert np.count_nonzero(qt["scales"].max(axis=1) == want) < 42 // 2


def test_row_scope_power_of_two_row_scaling():
    """Multiplying one row by 2^k (exact in bf16 and fp32) multiplies only
    that row's amax and s_dec by 2^k and leaves every code and block scale
    unchanged: the row's global scale absorbs the factor exactly."""
    x = _rows_over_decades(16, 128, 13)
    f = F.bf16_bits_to_f32(x)
    q = Q.quantize(x, "nvfp4", scope="row")
    for r, k in ((3, 7), (9, -5)):
        g = f.copy()
        g[r] *= np.float32(2.0 ** k)
        q2 = Q.quantize(bits(g), "nvfp4", scope="row")
        assert np.array_equal(q2["codes"], q["codes"])
        assert np.array_equal(q2["scales"], q["scales"])
        want = q["s_dec"].copy()
        want[r] = np.float32(want[r] * np.float32(2.0 ** k))
        assert np.array_equal(q2["s_dec"], want)
        assert q2["amax"][r] == np.float32(q["amax"][r] * np.float32(2.0 ** k))


def test_row_scope_keeps_small_rows_that_the_tensor_scale_loses():
    """Rows 2^40 below the tensor amax fall under the E4M3 scale range with
    one tensor scale (their block scales underflow to 0 and the rows decode
    to 0); with per-row scales no block underflows and every row decodes
    within the NVFP4 error (relative Frobenius error below 0.15)."""
    R, C = 21, 64
    x = _rows_over_decades(R, C, 14)
    f = F.bf16_bits_to_f32(x).astype(np.float64)
    qr = Q.quantize(x, "nvfp4", scope="row")
    qt = Q.quantize(x, "nvfp4")
    assert qr["counters"]["scale_underflow"] == 0
    assert qt["counters"]["scale_underflow"] > 0
    vr = Q.dequantize(qr["codes"], qr["scales"], "nvfp4", "1d", qr["s_dec"], R, C)
    vt = Q.dequantize(qt["codes"], qt["scales"], "nvfp4", "1d", qt["s_dec"], R, C)
    err_r = np.linalg.norm(vr - f, axis=1) / np.linalg.norm(f, axis=1)
    err_t = np.linalg.norm(vt - f, axis=1) / np.linalg.norm(f, axis=1)
    assert np.all(err_r < 0.15), err_r
    assert err_t[0] == 1.0          # row 0 (scale 2^-20) decodes to all zeros
