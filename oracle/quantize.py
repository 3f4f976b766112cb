"""FP4 block-scaled quantization, dequantization and event counters.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The steps follow App. B of "Pretraining Large Language Models with NVFP4"
in the order the page gives them; the display equations were lost from the
page, so each is restated from its surrounding prose:

  B.1 (Eq. 1)  tensor amax, global encode scale s_enc = 6 * 448 / amax, and
               global decode scale s_dec = 1 / s_enc, both fp32.  The UE5M3
               recipe (arXiv 2609.02846) replaces 448 by a target T and may
               use a stale tensor amax refreshed periodically.
  B.2 (Eq. 2)  local decode scale s_dec_L = amax_B / 6.
      (Eq. 3)  scale code = RNE(s_dec_L * s_enc) in the block-scale format;
               local encode scale s_enc_L = 1 / (fp32(scale) * s_dec).
  B.3 (Eq. 4)  element code = Q(x * s_enc_L), Q = E2M1 conversion.
  B.4          MXFP4: power-of-two UE8M0 scale rounded up so the block amax
               never saturates; no tensor scale.
  MXFP8        (2D-block FP4 page: the Q/K projections stay in MXFP8) E4M3
               elements in 1x32 blocks with a UE8M0 scale, read as the OCP
               MX format with B.4's round-up rule (B.4 names saturation as the
               MXFP8 convergence problem it avoids): 2^e with e the smallest
               integer such that 448 * 2^e >= amax_B; element code = sign bit
               7 | E4M3 RNE code of |x * 2^-e|; one byte per element.
  B.1 (end)    the "global" scale may cover a smaller span than the tensor,
               a row for instance, so that no separate pass over memory is
               needed for the amax: scope="row" gives every row of the
               output code matrix its own amax, s_enc and s_dec (Eq. 1 per
               row); each row is then quantized exactly as a one-row tensor.
  §4.3         2D weights: one scale per 16x16 tile (16 in x 16 out channels).
  §4.4         stochastic rounding on gradients: round to one of the two
               neighbours with probability inversely proportional to the
               distance.

Arithmetic is fp32 with correctly rounded division, no fused multiply-add,
in exactly the order above.  Readings of points the pages leave open (each
also listed in the design notes):
  * 6 * T is formed in fp32 (exact for T = 448 and 2048).
  * amax = 0 gives s_enc = 1; an s_enc or s_enc_L that overflows fp32 is
    clamped to the largest finite fp32 value.  A zero scale code gives
    s_enc_L = 0, so every code of that block is +-0.
  * Scale conversion saturates at the format maximum (448 for E4M3, 122880
    for UE5M3) and never yields NaN.
  * E2M1 conversion saturates |y| > 6 to 6, also under stochastic rounding.
  * The code's sign bit is the sign bit of y = x * s_enc_L.
  * Stochastic rounding: lo = largest E2M1 magnitude <= |y|, hi = the next
    one, f = (|y| - lo)/(hi - lo) in [0, 1); with 16 random bits r, round up
    iff r + floor(65536 f) >= 65536, i.e. when the random bits, added to the
    first 16 bits of the fraction f, carry.  This rounds up with probability
    floor(65536 f) / 65536, within 2^-16 of f.  Random bits come from
    ``philox.sr_random16`` keyed by the element's index in the OUTPUT layout
    (r * C + c for the [R, C] code matrix).
  * Packing: byte j of a code row holds element 2j in its low nibble and
    element 2j + 1 in its high nibble.  Scales are row-major [R, C / BS];
    2D scales are [R / 16, C / 16]; colwise output is the transposed matrix.

Counters (events named by the UE5M3 abstract: block-scale saturation and
underflow; the exact definitions are a reading):
  scale_saturated  s_dec_L * s_enc exceeds the scale format maximum
  scale_underflow  amax_B > 0 but the scale code is 0
  scale_subnormal  the scale code is a nonzero subnormal (exponent field 0)
  elem_saturated   |y| > 6
  elem_underflow   the quantized value is nonzero but its code is +-0
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from .philox import sr_random16
from .rht import rht_cols

FLT_MAX = np.float32(np.finfo(np.float32).max)

FORMATS = ("nvfp4", "ue5m3", "mxfp4", "mxfp8")
BLOCK = {"nvfp4": 16, "ue5m3": 16, "mxfp4": 32, "mxfp8": 32}
ELEM_MAX = {"mxfp4": 6.0, "mxfp8": 448.0}        # largest element magnitude of an MX format
COUNTERS = ("scale_saturated", "scale_underflow", "scale_subnormal",
            "elem_saturated", "elem_underflow")


def zero_counters():
    return {k: 0 for k in COUNTERS}


# ------------------------------------------------------------ B.1 -------
def tensor_amax(v):
    """amax_X = max |x| over the tensor, as fp32 (App. B.1)."""
    v = np.asarray(v, dtype=np.float32)
    if v.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(v)))


def row_amax(v):
    """max |x| of every row (fp32 [R]): the amax of the per-row global
    scale (App. B.1, last sentence); 0 for an empty row."""
    v = np.asarray(v, dtype=np.float32)
    if v.shape[1] == 0:
        return np.zeros(v.shape[0], np.float32)
    return np.max(np.abs(v), axis=1).astype(np.float32)


def global_scales(amax, target=448.0):
    """(s_enc_G, s_dec_G) from the tensor amax (App. B.1, Eq. 1), fp32."""
    amax = np.float32(amax)
    six_t = np.float32(6.0) * np.float32(target)
    with np.errstate(over="ignore", divide="ignore"):
        s_enc = np.float32(1.0) if amax == 0 else np.float32(six_t / amax)
    if not np.isfinite(s_enc):
        s_enc = FLT_MAX
    s_dec = np.float32(np.float32(1.0) / s_enc)
    return s_enc, s_dec


# ------------------------------------------------------------ B.2 -------
def block_scales_two_level(amax_b, s_enc_g, s_dec_g, fmt, scale_round="rne"):
    """Scale codes and local encode scales for NVFP4 / UE5M3 blocks.

    amax_b: fp32 array of block amaxes.  scale_round: "rne" (App. B.2: the
    scale is rounded to nearest) or "up" (the 2D-block page's truncation-free
    scaling, read as: the scale is rounded up, so the block amax times the
    encode scale does not exceed 6 and no element is clipped).  Returns
    (codes uint8, s_enc_L fp32, per-block event arrays dict).
    """
    assert scale_round in ("rne", "up")
    amax_b = np.asarray(amax_b, dtype=np.float32)
    s_dec_l = (amax_b / np.float32(6.0)).astype(np.float32)            # Eq. 2
    with np.errstate(over="ignore"):
        t = (s_dec_l * np.float32(s_enc_g)).astype(np.float32)          # Eq. 3
    t = np.where(np.isfinite(t), t, FLT_MAX).astype(np.float32)
    if fmt == "nvfp4":
        code, sat = (F.e4m3_up_sat if scale_round == "up" else F.e4m3_rne_sat)(t)
        s_hat = F.e4m3_value(code).astype(np.float32)
    elif fmt == "ue5m3":
        code, sat = (F.ue5m3_up_sat if scale_round == "up" else F.ue5m3_rne_sat)(t)
        s_hat = F.ue5m3_value(code).astype(np.float32)
    else:
        raise ValueError(fmt)
    p = (s_hat * np.float32(s_dec_g)).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        inv = (np.float32(1.0) / p).astype(np.float32)
    inv = np.minimum(inv, FLT_MAX)
    s_enc_l = np.where(code == 0, np.float32(0.0), inv).astype(np.float32)
    events = {
        "scale_saturated": sat,
        "scale_underflow": (amax_b > 0) & (code == 0),
        "scale_subnormal": (code >= 1) & (code <= 7),
    }
    return code, s_enc_l, events


# ------------------------------------------------------------ B.4 -------
def block_scales_mx(amax_b, elem_max=6.0):
    """UE8M0 codes and encode scales for MX blocks (App. B.4, §3).

    The decode scale is the smallest power of two 2^e with elem_max * 2^e >=
    amax_B (rounded up so the block amax never saturates; elem_max = 6 for
    MXFP4's E2M1, 448 for MXFP8's E4M3), e clamped to [-127, 127]; an
    all-zero block takes e = -127.  Encode scale = 2^-e.
    """
    a = np.asarray(amax_b, dtype=np.float32).astype(np.float64)
    e = np.full(a.shape, -127, dtype=np.int64)
    nz = a > 0
    # exact search: start from a float estimate, then fix with exact tests
    est = np.zeros(a.shape, dtype=np.int64)
    est[nz] = np.ceil(np.log2(a[nz] / elem_max)).astype(np.int64)
    for _ in range(3):
        too_small = nz & (elem_max * np.ldexp(1.0, est) < a)
        est = np.where(too_small, est + 1, est)
        can_lower = nz & (elem_max * np.ldexp(1.0, est - 1) >= a)
        est = np.where(can_lower, est - 1, est)
    e[nz] = est[nz]
    e = np.clip(e, -127, 127)
    code = (e + 127).astype(np.uint8)
    s_enc_l = np.ldexp(1.0, -e).astype(np.float32)
    events = {k: np.zeros(a.shape, dtype=bool)
              for k in ("scale_saturated", "scale_underflow", "scale_subnormal")}
    return code, s_enc_l, events


# ------------------------------------------------------------ B.3 -------
def encode_elements(v, s_enc_l, rnd="rne", r16=None):
    """E2M1 codes of v * s_enc_L (App. B.3, Eq. 4) with RNE or SR (§4.4).

    v: fp32 [..., n]; s_enc_l: fp32 broadcastable to v; r16: uint16 like v
    (SR only).  Returns (codes uint8, elem_saturated bool, elem_underflow bool).
    """
    v = np.asarray(v, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (v * np.asarray(s_enc_l, dtype=np.float32)).astype(np.float32)
    m = np.abs(y.astype(np.float64))
    sat = m > F.E2M1_MAX
    if rnd == "rne":
        code, _ = F.e2m1_rne(y)
    elif rnd == "sr":
        assert r16 is not None and r16.shape == v.shape
        mc = np.minimum(m, F.E2M1_MAX)
        lo = F.e2m1_floor_code(mc)
        top = lo >= 7
        lo_c = np.minimum(lo, 6)
        lo_v = F.E2M1_MAG[lo_c]
        hi_v = F.E2M1_MAG[lo_c + 1]
        # fp32 arithmetic, exact: (m - lo) by Sterbenz, division by a power of 2
        frac = ((mc.astype(np.float32) - lo_v.astype(np.float32))
                / (hi_v - lo_v).astype(np.float32)).astype(np.float32)
        lead16 = np.floor(frac.astype(np.float64) * 65536.0).astype(np.int64)
        up = r16.astype(np.int64) + lead16 >= 65536
        mag = np.where(top, 7, lo_c + up.astype(np.int64))
        code = (mag.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << 3))
    else:
        raise ValueError(rnd)
    under = (v != 0) & ((code & 7) == 0)
    return code.astype(np.uint8), sat, under


def encode_elements_e4m3(v, s_enc_l):
    """MXFP8 element codes of v * s_enc_L: y = fp32(v * s), code = sign bit 7 |
    E4M3 RNE code of |y| (saturating at 448, which the rounded-up block scale
    never reaches).  Returns (codes uint8, elem_saturated, elem_underflow)."""
    v = np.asarray(v, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (v * np.asarray(s_enc_l, dtype=np.float32)).astype(np.float32)
    mag, sat = F.e4m3_rne_sat(np.abs(y))
    code = mag.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << 7)
    under = (v != 0) & (mag == 0)
    return code, sat, under


def pack_codes(codes):
    """[R, C] nibbles -> [R, C/2] bytes, even element in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] % 2 == 0
    return (codes[..., 0::2] & 0xF) | ((codes[..., 1::2] & 0xF) << 4)


def unpack_codes(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# ------------------------------------------------------ full quantize ----
def quantize(x_bits, fmt="nvfp4", block="1d", orient="row", rnd="rne",
             seed=0, offset=0, rht=False, signs=0, target=448.0,
             amax=None, emit_transpose=False, index_base=0, rht_n=16, scale_round="rne",
             scope="tensor"):
    """Quantize a bf16 matrix (uint16 bit patterns, [R, C]).

    orient="row": blocks run along C; output codes [R, C/2], scales
    [R, C/BS].  orient="col": the matrix quantized is X^T, so output codes
    are [C, R/2] and scales [C, R/BS].  rht=True first rotates every group
    of 16 consecutive elements along the blocked axis -- 16 rows of a column
    for orient="col" (the Wgrad operands, App. C), 16 columns of a row for
    orient="row" (the Fprop / Dgrad operands, §4.2) -- by (1/4) D_r H16, and
    the tensor amax is taken after the rotation (rht_n: the size N of the
    variant transforms, groups of N elements, `signs` an N-bit mask).  block="2d":
    16x16 tiles of X (rowwise only); scales [R/16, C/16]; emit_transpose
    also returns the codes of X^T ([C, R/2]) quantized with the same tile
    scales.
    amax: None to compute it, or a given (possibly stale) fp32 amax.
    index_base: output-layout index of element (0, 0), so that a slab of
    output rows of a larger matrix draws the same random bits (SR only).
    scale_round: "rne" or "up" (truncation-free block scales; two-level
    formats -- MXFP4 scales are always rounded up).  block="2d" with SR
    draws the random bits of element (r, c) of X at index r*C + c, so the
    codes of X^T are exactly the transposed codes of X.
    scope: "tensor" (one global scale) or "row" (two-level formats, 1D: one
    global scale per row of the output code matrix; `amax`, if given, and
    the returned amax and s_dec are then fp32 arrays with one entry per row).

    Returns a dict: codes, scales, codes_t (2D only), amax, s_dec, counters.
    """
    assert fmt in FORMATS and block in ("1d", "2d") and orient in ("row", "col")
    assert rnd in ("rne", "sr") and scope in ("tensor", "row")
    mx = fmt in ("mxfp4", "mxfp8")
    assert scope == "tensor" or (not mx and block == "1d")
    if fmt == "mxfp8":
        assert block == "1d" and rnd == "rne" and not rht
    x = F.bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16))
    assert x.ndim == 2
    R, C = x.shape
    bs = BLOCK[fmt]
    if block == "2d":
        assert not mx and orient == "row" and not rht
        assert R % 16 == 0 and C % 16 == 0
        bs = 16
    if rht:
        if orient == "col":
            assert R % rht_n == 0
            x = rht_cols(x, signs, rht_n)
        else:      # along the rows: the columns of X^T
            assert C % rht_n == 0
            x = rht_cols(x.T, signs, rht_n).T.copy()
    v = x.T.copy() if orient == "col" else x               # rows of v are blocked
    Ro, Co = v.shape
    assert Co % bs == 0, "block axis must be a multiple of the block size"

    if mx:
        assert amax is None, "MX formats have no tensor scale"
        amax_x, s_enc_g, s_dec_g = None, np.float32(1.0), np.float32(1.0)
    elif scope == "row":
        amax_x = (row_amax(v) if amax is None
                  else np.asarray(amax, dtype=np.float32).reshape(Ro).copy())
        pairs = [global_scales(a, target) for a in amax_x]
        s_enc_g = np.array([p[0] for p in pairs], np.float32).reshape(Ro, 1)
        s_dec_g = np.array([p[1] for p in pairs], np.float32).reshape(Ro, 1)
    else:
        amax_x = tensor_amax(v) if amax is None else np.float32(amax)
        s_enc_g, s_dec_g = global_scales(amax_x, target)

    # block amax
    if block == "1d":
        vb = v.reshape(Ro, Co // bs, bs)
        amax_b = (np.abs(vb).max(axis=2) if Ro * Co
                  else np.zeros((Ro, Co // bs), np.float32))
    else:
        vt = v.reshape(Ro // 16, 16, Co // 16, 16)
        amax_b = (np.abs(vt).max(axis=(1, 3)) if Ro * Co
                  else np.zeros((Ro // 16, Co // 16), np.float32))

    if mx:
        scode, s_enc_l, sev = block_scales_mx(amax_b, ELEM_MAX[fmt])
    else:
        scode, s_enc_l, sev = block_scales_two_level(amax_b, s_enc_g, s_dec_g, fmt, scale_round)

    # per-element encode scale
    if block == "1d":
        s_el = np.repeat(s_enc_l, bs, axis=1)
    else:
        s_el = np.repeat(np.repeat(s_enc_l, 16, axis=0), 16, axis=1)

    r16 = None
    if rnd == "sr":
        idx = (int(index_base) + np.arange(Ro, dtype=np.int64)[:, None] * Co
               + np.arange(Co, dtype=np.int64)[None, :])
        r16 = sr_random16(idx, seed, offset)
    if fmt == "mxfp8":
        codes, esat, eund = encode_elements_e4m3(v, s_el)
    else:
        codes, esat, eund = encode_elements(v, s_el, rnd, r16)

    counters = {
        "scale_saturated": int(np.count_nonzero(sev["scale_saturated"])),
        "scale_underflow": int(np.count_nonzero(sev["scale_underflow"])),
        "scale_subnormal": int(np.count_nonzero(sev["scale_subnormal"])),
        "elem_saturated": int(np.count_nonzero(esat)),
        "elem_underflow": int(np.count_nonzero(eund)),
    }
    out = {
        "codes": codes if fmt == "mxfp8" else pack_codes(codes),   # MXFP8: a byte each
        "scales": scode.astype(np.uint8),
        "amax": (None if amax_x is None else
                 amax_x if scope == "row" else np.float32(amax_x)),
        "s_dec": s_dec_g.reshape(Ro) if scope == "row" else np.float32(s_dec_g),
        "counters": counters,
        "codes_unpacked": codes,
    }
    if block == "2d" and emit_transpose:
        out["codes_t"] = pack_codes(codes.T.copy())
    return out


# --------------------------------------------------------- dequantize ----
def scale_values(scodes, fmt):
    """Decoded block-scale values as float64 (exact)."""
    if fmt == "nvfp4":
        return F.e4m3_value(scodes)
    if fmt == "ue5m3":
        return F.ue5m3_value(scodes)
    return F.ue8m0_value(scodes)


def element_values(codes, fmt, R, C):
    """Element values (float64, exact) of an [R, C] code matrix: packed E2M1
    ([R, C/2] bytes) or MXFP8's E4M3 bytes ([R, C], sign in bit 7)."""
    if fmt == "mxfp8":
        c = np.asarray(codes, dtype=np.uint8).reshape(R, C).astype(np.int64)
        mag = F.e4m3_value(c & 0x7F)
        return np.where(c & 0x80, -mag, mag)
    return F.e2m1_value(unpack_codes(np.asarray(codes, dtype=np.uint8).reshape(R, C // 2)))


def element_scales(scodes, fmt, block, R, C):
    """Per-element block-scale values (float64) for an [R, C] code matrix."""
    sv = scale_values(scodes, fmt)
    if block == "1d":
        bs = BLOCK[fmt]
        return np.repeat(sv.reshape(R, C // bs), bs, axis=1)
    return np.repeat(np.repeat(sv.reshape(R // 16, C // 16), 16, axis=0), 16, axis=1)


def dequantize(codes_packed, scodes, fmt, block, s_dec, R, C, out="f32"):
    """v = fp32(fp32(e2m1 * scale) * s_dec_G); bf16 output rounds v (RNE).

    The decode follows App. B.2-B.3 of the NVFP4 paper (the decode scales
    undo the encode scales).  element * scale is exact in fp32 (E2M1, or
    MXFP8's E4M3 times a power of two).  MX formats have no tensor scale
    (s_dec is taken as 1).  s_dec may be an array of R per-row decode scales
    (scope="row").
    """
    e = element_values(codes_packed, fmt, R, C)
    s = element_scales(scodes, fmt, block, R, C)
    with np.errstate(over="ignore"):
        prod = (e * s).astype(np.float32)
        if fmt in ("mxfp4", "mxfp8"):
            sd = np.float32(1.0)
        elif np.ndim(s_dec) == 0:
            sd = np.float32(s_dec)
        else:
            sd = np.asarray(s_dec, dtype=np.float32).reshape(R, 1)
        v = (prod * sd).astype(np.float32)
    if out == "bf16":
        return F.f32_to_bf16_bits(v)
    return v


def operand_values(codes_packed, scodes, fmt, block, R, K):
    """Exact element values e2m1 * scale (float64) of a GEMM operand [R, K],
    without the tensor scale (it is applied after the GEMM, App. B.3)."""
    return element_values(codes_packed, fmt, R, K) * element_scales(scodes, fmt, block, R, K)
