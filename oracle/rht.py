"""Random Hadamard transform (RHT) applied to Wgrad inputs: 16-point, and
the N-point variants N in {4, 16, 32, 64, 128}.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

NVFP4 pretraining paper, §4.2 and App. C: the transform multiplies each
16-element tile by H_r = D_r H, where H is the Sylvester Hadamard matrix and
D_r a random diagonal of signs that flips whole rows of H; it is applied to
both Wgrad operands so the rotation cancels in the dot product, and the
quantization scale is computed in the rotated space.

Readings (the page's formulas were lost, the implementation paragraph is cut):
  * H16 has +-1 entries (H H^T = 16 I); the applied map is (1/4) D_r H16,
    which is orthonormal.
  * The 16-vector is 16 consecutive tokens of one feature column.
  * Arithmetic is fp32, as a fast Walsh-Hadamard transform whose butterfly
    stages run with stride 1, 2, 4, 8 in that order; each butterfly maps
    (a, b) to (a + b, a - b); then every entry is multiplied by 1/4 (exact),
    then entry i is negated if bit i of the sign mask is set.
  * Size N (the page weighs N = 4, 16 and 128 and picks 16, §4.2): the same
    steps with strides 1, 2, ..., N/2, the scale fl32(1/sqrt(N)) (exact for
    N = 4, 16, 64; for N = 32 and 128 the fp32 number nearest to
    sqrt(2)/8 and sqrt(2)/16), and an N-bit sign mask.  The N-vector is N
    consecutive tokens of one feature column.
"""
from __future__ import annotations

import numpy as np


def fwht16_f32(v):
    """Unnormalized Walsh-Hadamard transform of the last axis (length 16), fp32.

    Equals v @ H16^T with H16[i, j] = (-1)^popcount(i & j), rounded after each
    butterfly stage.
    """
    v = np.array(v, dtype=np.float32, copy=True)
    assert v.shape[-1] == 16
    for h in (1, 2, 4, 8):
        out = v.copy()
        for i in range(16):
            if i & h == 0:
                a, b = v[..., i], v[..., i + h]
                out[..., i] = a + b
                out[..., i + h] = a - b
        v = out
    return v


def rht16_vec(v, signs):
    """(1/4) D_r H16 v on the last axis (length 16), in fp32."""
    y = fwht16_f32(v) * np.float32(0.25)
    flip = np.array([(signs >> i) & 1 for i in range(16)], dtype=bool)
    y[..., flip] = -y[..., flip]
    return y


def rht16_cols(x, signs):
    """Transform every column of x [R, C] (fp32) in groups of 16 rows.

    Rows 16g..16g+15 of column c form one vector.  R must be a multiple of 16.
    Returns fp32 [R, C].
    """
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert R % 16 == 0
    v = x.reshape(R // 16, 16, C).transpose(0, 2, 1)        # [G, C, 16]
    y = rht16_vec(v, signs)
    return y.transpose(0, 2, 1).reshape(R, C)


SIZES = (4, 16, 32, 64, 128)


def rht_scale(n):
    """fl32(1 / sqrt(n)): the fp32 number nearest to 1/sqrt(n)."""
    assert n in SIZES
    return np.float32(1.0 / np.sqrt(np.float64(n)))


def fwht_f32(v, n):
    """Unnormalized Walsh-Hadamard transform of the last axis (length n),
    fp32, butterfly strides 1, 2, ..., n/2 in that order."""
    v = np.array(v, dtype=np.float32, copy=True)
    assert v.shape[-1] == n and n in SIZES
    h = 1
    while h < n:
        out = v.copy()
        for i in range(n):
            if i & h == 0:
                a, b = v[..., i], v[..., i + h]
                out[..., i] = a + b
                out[..., i + h] = a - b
        v = out
        h *= 2
    return v


def rht_vec(v, signs, n):
    """fl32(1/sqrt(n)) D_r H_n v on the last axis (length n), in fp32;
    bit i of the integer `signs` negates output entry i."""
    y = fwht_f32(v, n) * rht_scale(n)
    flip = np.array([(int(signs) >> i) & 1 for i in range(n)], dtype=bool)
    y[..., flip] = -y[..., flip]
    return y


def rht_cols(x, signs, n=16):
    """Transform every column of x [R, C] (fp32) in groups of n rows.
    R must be a multiple of n.  Returns fp32 [R, C]."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert R % n == 0
    v = x.reshape(R // n, n, C).transpose(0, 2, 1)        # [G, C, n]
    y = rht_vec(v, signs, n)
    return y.transpose(0, 2, 1).reshape(R, C)
