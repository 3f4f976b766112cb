"""Philox4x32-10 counter-based random numbers, as the stochastic-rounding source.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Philox4x32 is defined in J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel
random numbers: as easy as 1, 2, 3" (SC'11): a 128-bit counter (c0..c3) and a
64-bit key (k0, k1); one round multiplies c0 and c2 by two fixed odd
constants, and the new counter is built from the high and low halves of the
two 64-bit products xor-ed with the other counter words and the key.  The key
is advanced by two Weyl constants between rounds; ten rounds make the
"-10" variant.

The NVFP4 pretraining paper (§4.4) only fixes what stochastic rounding must
do (probability of rounding to a neighbour inversely proportional to the
distance); the generator and its keying are a reading: key = seed, counter =
(element_index >> 3, offset), 16 random bits per element.
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox4x32 rounds on counter arrays (uint32-valued) with key (k0, k1).

    Counter words may be arrays (broadcast together); the key is scalar.
    Returns four uint32 arrays.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & _MASK32 for c in (c0, c1, c2, c3))
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
        p0 = PHILOX_M0 * c0            # < 2^64, exact in uint64
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0)
    return tuple(c.astype(np.uint32) for c in (c0, c1, c2, c3))


def sr_random16(idx, seed, offset):
    """16 random bits for each element index ``idx`` (int64 array).

    Philox4x32-10 with key = (seed low, seed high) and counter =
    (g low, g high, offset low, offset high), g = idx >> 3.  The 128 output
    bits serve 8 consecutive indices: index j = idx & 7 takes a 16-bit half
    of output word j >> 1, the upper half for even j and the lower half for
    odd j.
    """
    idx = np.asarray(idx, dtype=np.int64)
    g = (idx >> 3).astype(np.uint64)
    seed = int(seed)
    offset = int(offset)
    words = philox4x32_10(g & _MASK32, g >> np.uint64(32),
                          np.uint64(offset & 0xFFFFFFFF), np.uint64((offset >> 32) & 0xFFFFFFFF),
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = np.stack(words, axis=-1)                      # [..., 4] uint32
    j = (idx & 7).astype(np.int64)
    word = np.take_along_axis(w.reshape(-1, 4), (j >> 1).reshape(-1, 1), axis=1).reshape(idx.shape)
    return ((word >> ((1 - (j & 1)) * 16).astype(np.uint32)) & 0xFFFF).astype(np.uint16)

