"""Pins of the oracle's 16-point random Hadamard transform."""
import numpy as np

import oracle as O


def _sylvester(n):
    """H_n by the Kronecker recursion H_2n = H_2 (x) H_n (unnormalised, +-1)."""
    h = np.array([[1.0]])
    h2 = np.array([[1.0, 1.0], [1.0, -1.0]])
    while h.shape[0] < n:
        h = np.kron(h2, h)
    return h


def _rht_matrix(signs):
    """Apply the oracle transform to the unit vectors: row i is e_i S H."""
    eye = np.eye(16, dtype=np.float32)
    return O.rht16(eye, signs).astype(np.float64)


def test_hadamard_is_sylvester_and_orthogonal():
    H = _rht_matrix(0) * 4.0
    assert np.array_equal(H, _sylvester(16))
    assert np.array_equal(H @ H.T, 16.0 * np.eye(16))
    Hn = _rht_matrix(0)
    assert np.allclose(Hn @ Hn.T, np.eye(16), atol=0)


def test_sign_flips_rows():
    s = 0b1010011100010110
    M = _rht_matrix(s)
    S = np.diag([-1.0 if (s >> i) & 1 else 1.0 for i in range(16)])
    assert np.array_equal(M, S @ (_sylvester(16) / 4.0))
    assert np.allclose(M @ M.T, np.eye(16), atol=0)


def test_butterfly_equals_matrix_product():
    rng = np.random.default_rng(3)
    s = 0xBEEF
    M = _rht_matrix(s)
    # small integers: every butterfly sum is exact, so bit-exact equality
    xi = rng.integers(-1000, 1000, size=(64, 16)).astype(np.float32)
    assert np.array_equal(O.rht16(xi, s).astype(np.float64), xi.astype(np.float64) @ M)
    # general values: equal to the FP64 product within FP32 rounding
    x = rng.standard_normal((4096, 16)).astype(np.float32)
    y = O.rht16(x, s).astype(np.float64)
    ref = x.astype(np.float64) @ M
    assert np.max(np.abs(y - ref)) < 4 * 2.0 ** -24 * np.max(np.abs(x)) * 4


def test_inverse_and_norm():
    rng = np.random.default_rng(4)
    s = 0x1234
    xi = rng.integers(-500, 500, size=(32, 16)).astype(np.float32)
    y = O.rht16(xi, s)
    back = O.rht16(y, 0)                      # H is its own inverse
    flip = np.array([-1.0 if (s >> i) & 1 else 1.0 for i in range(16)], np.float32)
    assert np.array_equal(back * flip, xi)
    x = rng.standard_normal((1000, 16)).astype(np.float32)
    y = O.rht16(x, s)
    n0 = np.linalg.norm(x.astype(np.float64), axis=1)
    n1 = np.linalg.norm(y.astype(np.float64), axis=1)
    assert np.max(np.abs(n1 - n0) / n0) < 1e-6


def test_transform_cancels_in_a_product():
    # (A H)(H^T B): the same orthogonal transform on both operands along the
    # contraction dim leaves A B^T unchanged.
    rng = np.random.default_rng(5)
    A = rng.standard_normal((24, 64)).astype(np.float32)
    B = rng.standard_normal((40, 64)).astype(np.float32)
    s = 0x5A5A
    At = O.rht16(A, s).astype(np.float64)
    Bt = O.rht16(B, s).astype(np.float64)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    assert np.max(np.abs(At @ Bt.T - ref)) < 1e-4


def test_rht_spreads_an_outlier():
    x = np.zeros((1, 16), np.float32)
    x[0, 5] = 100.0
    y = O.rht16(x, 0x0F0F)
    assert np.all(np.abs(y) == 25.0)          # 100 / sqrt(16) into every output
