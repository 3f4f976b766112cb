"""Pins for oracle/rht.py: the 16-point randomized Hadamard transform.

Checked against scipy.linalg.hadamard (Sylvester construction, a library
routine), the orthogonality the NVFP4 paper relies on (App. C: the rotation
of each operand cancels in the product), closed forms, and an fp64 error
bound for the fp32 butterflies.
"""
import numpy as np
import scipy.linalg

from oracle import rht as R
from fp4_block_scaled_x16_amd import inputs

H16 = scipy.linalg.hadamard(16).astype(np.float64)


def test_fwht_of_one_hot_is_hadamard_column():
    eye = np.eye(16, dtype=np.float32)
    got = R.fwht16_f32(eye)                 # row j = transform of e_j
    assert np.array_equal(got.astype(np.float64), H16.T)
    assert np.array_equal(H16 @ H16.T, 16 * np.eye(16))


def test_signs_flip_output_rows():
    # H_r = D_r H: bit i of the mask negates OUTPUT entry i (a row of H)
    signs = 0b1010000000000101
    d = np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])
    got = R.rht16_vec(np.eye(16, dtype=np.float32), signs).astype(np.float64)
    want = (0.25 * np.diag(d) @ H16).T       # row j = (1/4) D H e_j
    assert np.array_equal(got, want)
    # orthonormal: M M^T = I exactly
    M = got.T
    assert np.array_equal(M @ M.T, np.eye(16))


def test_constant_vector_concentrates():
    c = np.float32(3.25)
    for signs in (0, 1, inputs.rht_sign_mask()):
        y = R.rht16_vec(np.full(16, c, np.float32), signs)
        want = np.zeros(16, np.float32)
        want[0] = -4 * c if signs & 1 else 4 * c
        assert np.array_equal(y, want)


def test_fp32_error_bound_against_fp64():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((20000, 16)) * 10.0 ** rng.uniform(-6, 6, (20000, 1))).astype(np.float32)
    signs = inputs.rht_sign_mask()
    d = np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])
    exact = (v.astype(np.float64) @ H16.T) * 0.25 * d
    got = R.rht16_vec(v, signs).astype(np.float64)
    bound = 4 * 2.0 ** -24 * 0.25 * np.abs(v.astype(np.float64)).sum(axis=1, keepdims=True)
    assert np.all(np.abs(got - exact) <= bound)


def test_cols_layout_and_cancellation():
    rng = np.random.default_rng(9)
    T, a, b = 64, 5, 7
    x = rng.standard_normal((T, a)).astype(np.float32)
    dy = rng.standard_normal((T, b)).astype(np.float32)
    s = inputs.rht_sign_mask()
    rx, rdy = R.rht16_cols(x, s), R.rht16_cols(dy, s)
    # each 16-row group of each column is transformed independently
    assert np.array_equal(rx[16:32, 3], R.rht16_vec(x[16:32, 3], s))
    # Wgrad with both operands rotated equals the unrotated product (App. C)
    lhs = rdy.astype(np.float64).T @ rx.astype(np.float64)
    rhs = dy.astype(np.float64).T @ x.astype(np.float64)
    assert np.allclose(lhs, rhs, rtol=1e-5, atol=1e-5)


# ------------------------------------------- N-point variants (N = 4 ... 128)
import fractions
import pytest


@pytest.mark.parametrize("n", R.SIZES)
def test_fwht_n_of_one_hot_is_hadamard_column(n):
    H = scipy.linalg.hadamard(n).astype(np.float64)
    got = R.fwht_f32(np.eye(n, dtype=np.float32), n).astype(np.float64)
    assert np.array_equal(got, H.T)
    assert np.array_equal(H @ H.T, n * np.eye(n))


def test_n16_variant_is_the_16_point_transform():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((500, 16)).astype(np.float32)
    s = inputs.rht_sign_mask()
    assert np.array_equal(R.rht_vec(v, s, 16), R.rht16_vec(v, s))
    x = rng.standard_normal((64, 9)).astype(np.float32)
    assert np.array_equal(R.rht_cols(x, s, 16), R.rht16_cols(x, s))


@pytest.mark.parametrize("n", R.SIZES)
def test_scale_is_nearest_fp32_to_inverse_sqrt(n):
    # exact rational check: no fp32 number lies closer to 1/sqrt(n)
    s = R.rht_scale(n)
    up, dn = np.nextafter(s, np.float32(1)), np.nextafter(s, np.float32(0))
    f = lambda x: fractions.Fraction(float(x))
    # |s - 1/sqrt(n)| <= |t - 1/sqrt(n)| for both neighbours t  <=>  compare squares
    def dist2_ok(t):
        # (s^2 - 1/n) and (t^2 - 1/n) sign-aware comparison via midpoint m:
        # s is nearest iff 1/n lies between the squares of the midpoints
        m = (f(s) + f(t)) / 2
        return (m * m - fractions.Fraction(1, n)) * (f(t) - f(s)) > 0
    assert dist2_ok(up) and dist2_ok(dn)
    if n in (4, 16, 64):
        assert f(s) * f(s) == fractions.Fraction(1, n)


@pytest.mark.parametrize("n", R.SIZES)
def test_signs_flip_rows_and_bound_against_fp64(n):
    H = scipy.linalg.hadamard(n).astype(np.float64)
    s = inputs.rht_sign_bits(n)
    d = np.array([-1.0 if (s >> i) & 1 else 1.0 for i in range(n)])
    scale = float(R.rht_scale(n))
    # one-hot inputs: exact
    got = R.rht_vec(np.eye(n, dtype=np.float32), s, n).astype(np.float64)
    assert np.array_equal(got, (scale * np.diag(d) @ H).T)
    # random inputs: log2(n) rounded stages plus the rounded scale
    rng = np.random.default_rng(n)
    v = (rng.standard_normal((4000, n)) * 10.0 ** rng.uniform(-6, 6, (4000, 1))).astype(np.float32)
    exact = (v.astype(np.float64) @ H.T) * scale * d
    stages = int(np.log2(n)) + 1
    bound = stages * 2.0 ** -24 * scale * np.abs(v.astype(np.float64)).sum(axis=1, keepdims=True)
    assert np.all(np.abs(R.rht_vec(v, s, n).astype(np.float64) - exact) <= bound)


@pytest.mark.parametrize("n", R.SIZES)
def test_n_point_cols_layout_and_cancellation(n):
    rng = np.random.default_rng(11 + n)
    T, a, b = 2 * n, 5, 7
    x = rng.standard_normal((T, a)).astype(np.float32)
    dy = rng.standard_normal((T, b)).astype(np.float32)
    s = inputs.rht_sign_bits(n)
    rx, rdy = R.rht_cols(x, s, n), R.rht_cols(dy, s, n)
    assert np.array_equal(rx[n:2 * n, 3], R.rht_vec(x[n:2 * n, 3], s, n))
    # (c D H)^T (c D H) = c^2 n I: the rotated Wgrad equals the plain one up
    # to the factor c^2 n (1 exactly when c^2 = 1/n)
    c2n = float(R.rht_scale(n)) ** 2 * n
    lhs = rdy.astype(np.float64).T @ rx.astype(np.float64)
    rhs = dy.astype(np.float64).T @ x.astype(np.float64) * c2n
    assert np.allclose(lhs, rhs, rtol=1e-5, atol=1e-5)
    assert abs(c2n - 1.0) < 1e-7
