"""Seeded synthetic inputs shaped like the linears of the NVFP4 pretraining
paper's models (1.2B Transformer, 8B and 12B hybrid Mamba-Transformer, §5
setup), at sequence length 8192.

This module holds only random-number generation and the rounding of the
draws to bf16; none of the quantization method's arithmetic.  Both the HIP
path and the CPU oracle take their inputs from here.

Every tensor is drawn with NumPy's PCG64 from SeedSequence([cfg_seed,
tensor_id]) (tensor ids: X or A = 0, W = 1, dY = 2) in float32, then rounded
to bf16 (nearest, ties to even) and returned as uint16 bit patterns.

Distributions:
  activations  N(0, 1), with exactly round(0.001 * n) entries chosen
               uniformly without replacement and multiplied by 50 (outliers)
  weights      N(0, 0.02^2)
  gradients    |v| = 10^U, U ~ Uniform(-8, -2), sign +-1 with probability 1/2
"""
from __future__ import annotations

import numpy as np

X_ID, W_ID, DY_ID, SIGNS_ID = 0, 1, 2, 3
STALE_SEED_OFFSET = 50
RHT_SEED = 7

#: tokens x in, out x in, tokens x out for each workload
CONFIGS = {
    1: dict(name="tiny-256", tokens=256, d_in=256, d_out=256, fmt="nvfp4"),
    2: dict(name="1.2B-ffn-up", tokens=8192, d_in=2048, d_out=6144, fmt="nvfp4"),
    3: dict(name="12B-ffn-up-rht", tokens=8192, d_in=4608, d_out=12288, fmt="nvfp4"),
    4: dict(name="8B-ffn-up-ue5m3", tokens=8192, d_in=4096, d_out=21504, fmt="ue5m3"),
    5: dict(name="8B-ffn-up-mx-vs-nv", tokens=8192, d_in=4096, d_out=21504, fmt="mxfp4"),
}


def _rng(cfg_seed, tensor_id):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_seed, tensor_id])))


def to_bf16_bits(f32):
    """float32 -> bf16 bit patterns, round to nearest even (finite input)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def activations(shape, cfg_seed=0, tensor_id=X_ID, outliers=True):
    rng = _rng(cfg_seed, tensor_id)
    n = int(np.prod(shape))
    x = rng.standard_normal(n, dtype=np.float32)
    if outliers and n:
        k = int(round(0.001 * n))
        idx = rng.choice(n, size=k, replace=False)
        x[idx] *= np.float32(50.0)
    return to_bf16_bits(x).reshape(shape)


def weights(shape, cfg_seed=0, tensor_id=W_ID, sigma=0.02):
    rng = _rng(cfg_seed, tensor_id)
    n = int(np.prod(shape))
    w = rng.standard_normal(n, dtype=np.float32) * np.float32(sigma)
    return to_bf16_bits(w).reshape(shape)


def gradients(shape, cfg_seed=0, tensor_id=DY_ID, lo_exp=-8.0, hi_exp=-2.0):
    rng = _rng(cfg_seed, tensor_id)
    n = int(np.prod(shape))
    u = rng.random(n, dtype=np.float32)
    mag = np.power(np.float32(10.0), np.float32(lo_exp) + np.float32(hi_exp - lo_exp) * u,
                   dtype=np.float32)
    sign = rng.integers(0, 2, n, dtype=np.uint8)
    mag[sign == 1] *= np.float32(-1.0)
    return to_bf16_bits(mag).reshape(shape)


def rht_sign_mask(seed=RHT_SEED):
    """The random diagonal D_r of the 16-point RHT as a 16-bit mask (bit i set:
    output row i is negated).  One vector is shared by all layers and both
    Wgrad operands; it is drawn here, from the seed, and passed to both the
    kernels and the oracle."""
    return int(_rng(seed, SIGNS_ID).integers(0, 1 << 16))


def rht_sign_bits(n, seed=RHT_SEED):
    """The random diagonal D_r of the n-point RHT as an n-bit integer mask
    (bit i set: output row i is negated); n = 16 gives rht_sign_mask()."""
    if n == 16:
        return rht_sign_mask(seed)
    bits = _rng(seed, SIGNS_ID + 100 + n).integers(0, 2, size=n)
    return sum(int(b) << i for i, b in enumerate(bits))


def normal(shape, sigma=1.0, cfg_seed=0, tensor_id=X_ID):
    rng = _rng(cfg_seed, tensor_id)
    n = int(np.prod(shape))
    return to_bf16_bits(rng.standard_normal(n, dtype=np.float32) * np.float32(sigma)).reshape(shape)


def linear_tensors(cfg, cfg_seed=0, which=("X", "W", "dY")):
    """The X [tokens, in], W [out, in] and dY [tokens, out] of a workload.

    Workload 1 (the tiny one) draws A ~ N(0, 1) without outliers and W ~
    N(0, 0.02^2), and has no dY.
    """
    c = CONFIGS[cfg]
    out = {}
    if "X" in which:
        out["X"] = activations((c["tokens"], c["d_in"]), cfg_seed, X_ID, outliers=(cfg != 1))
    if "W" in which:
        out["W"] = weights((c["d_out"], c["d_in"]), cfg_seed, W_ID)
    if "dY" in which and cfg != 1:
        out["dY"] = gradients((c["tokens"], c["d_out"]), cfg_seed, DY_ID)
    return out
