"""Block-scaled GEMM reference (Fprop / Dgrad / Wgrad), fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

NVFP4 pretraining paper, App. B.3 (Eq. 5 prose): the matrix unit multiplies
each block's partial dot product by the two local decode scales and
accumulates; the global decode scales of both operands are applied to the
output after the GEMM.  §4.1 / Fig. 5: each linear layer runs three such
GEMMs (Fprop, Dgrad, Wgrad) on quantized inputs and writes BF16 or FP32.

Because every element value e2m1 * scale is a short dyadic rational, the
plain definition is used: D[m, n] = s_A * s_B * sum_k a[m, k] * b[n, k],
with the sum taken by a float64 matrix product and the result rounded once
to fp32.  (Scaling per block before or after the partial sums is the same
number in exact arithmetic.)

Layout: "TN" -- both operands are K-major: A is [M, K], B is [N, K].

Global decode scales are either one fp32 number per operand or, for the
per-row global scale (App. B.1, last sentence), one per operand row: s_A[m]
per row of A and s_B[n] per row of B, so D[m, n] takes s_A[m] * s_B[n].
"""
from __future__ import annotations

import numpy as np


def _scale(s_dec_a, s_dec_b):
    """s_A s_B in float64, shaped to broadcast over [M, N] (a scalar, or
    s_A as a column and s_B as a row when they are per-row vectors)."""
    sa = np.asarray(s_dec_a, dtype=np.float32).astype(np.float64)
    sb = np.asarray(s_dec_b, dtype=np.float32).astype(np.float64)
    if sa.ndim:
        sa = sa.reshape(-1, 1)
    if sb.ndim:
        sb = sb.reshape(1, -1)
    return sa * sb


def gemm_ref(a_vals, b_vals, s_dec_a=1.0, s_dec_b=1.0):
    """D = fp32(s_A * s_B * (A @ B^T)) with A, B float64 element values."""
    a = np.asarray(a_vals, dtype=np.float64)
    b = np.asarray(b_vals, dtype=np.float64)
    acc = a @ b.T
    with np.errstate(over="ignore"):
        return (acc * _scale(s_dec_a, s_dec_b)).astype(np.float32)


def gemm_abs_bound(a_vals, b_vals, s_dec_a=1.0, s_dec_b=1.0):
    """s_A * s_B * sum_k |a[m, k] * b[n, k]| (float64), the scale of the
    per-element tolerance |D_gpu - D_ref| <= 1e-5 * bound."""
    a = np.abs(np.asarray(a_vals, dtype=np.float64))
    b = np.abs(np.asarray(b_vals, dtype=np.float64))
    return (a @ b.T) * _scale(s_dec_a, s_dec_b)


def gemm_ref_entries(a_vals, b_vals, rows, cols, s_dec_a=1.0, s_dec_b=1.0):
    """Reference and bound for selected entries (rows[i], cols[i]) only."""
    a = np.asarray(a_vals, dtype=np.float64)[rows]
    b = np.asarray(b_vals, dtype=np.float64)[cols]
    sa = np.asarray(s_dec_a, dtype=np.float32).astype(np.float64)
    sb = np.asarray(s_dec_b, dtype=np.float32).astype(np.float64)
    s = (sa[rows] if sa.ndim else sa) * (sb[cols] if sb.ndim else sb)
    acc = np.einsum("ik,ik->i", a, b)
    bound = np.einsum("ik,ik->i", np.abs(a), np.abs(b)) * s
    with np.errstate(over="ignore"):
        return (acc * s).astype(np.float32), bound
