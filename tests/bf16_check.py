"""Check of a bf16 GEMM output against the oracle's fp64 result."""
import numpy as np

from oracle import formats as F

TOL = 1e-5


def bf16_close(got_bits, ref, bound):
    """A bf16 D is the fp32 result (within 1e-5 * bound of ref) rounded once
    to nearest: within that plus half a bf16 ulp of |ref| + 1e-5 * bound."""
    got = F.bf16_bits_to_f32(np.asarray(got_bits, np.uint16)).astype(np.float64)
    ref = np.asarray(ref, np.float64)
    mag = np.abs(ref) + TOL * bound
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 1e-300))) - 8)
    err = np.abs(got - ref)
    bad = err > TOL * bound + half_ulp
    assert not bad.any(), np.argwhere(bad)[:5].tolist()
