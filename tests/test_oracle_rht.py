"""Pins of the oracle's 16-point random Hadamard transform.

The oracle applies a butterfly; these tests recover the matrix it applies
from basis vectors and compare it with the Sylvester definition, check the
H H^T = 16 I identity, exactness on small integers, norm preservation, the
wgrad cancellation and the outlier spreading the pages describe.
"""
import numpy as np

import oracle
import workloads


def sylvester_h16():
    i = np.arange(16)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def test_h_times_ht_is_16_identity():
    H = sylvester_h16()
    np.testing.assert_array_equal(H @ H.T, 16 * np.eye(16))


def _oracle_matrix(mask):
    cols = [oracle.rht16(np.eye(16, dtype=np.float32)[j], mask) for j in range(16)]
    return np.stack(cols, axis=1).astype(np.float64)


def test_butterfly_applies_quarter_h_diag_s():
    H = sylvester_h16()
    for mask in (0, 0x0001, 0x8000, 0xA5A5, workloads.rht_sign_mask()):
        s = np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(16)])
        np.testing.assert_array_equal(_oracle_matrix(mask), 0.25 * H @ np.diag(s))


def test_small_integer_inputs_exact():
    H = sylvester_h16()
    rng = np.random.default_rng(5)
    mask = workloads.rht_sign_mask()
    s = np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(16)])
    for _ in range(200):
        x = rng.integers(-1000, 1000, 16).astype(np.float32)
        np.testing.assert_array_equal(oracle.rht16(x, mask).astype(np.float64),
                                      0.25 * H @ (s * x.astype(np.float64)))


def test_orthonormal_norm_preserved():
    rng = np.random.default_rng(6)
    for _ in range(200):
        x = rng.standard_normal(16).astype(np.float32)
        y = oracle.rht16(x, 0x1234).astype(np.float64)
        n0 = np.linalg.norm(x.astype(np.float64))
        assert abs(np.linalg.norm(y) - n0) <= 16 * 2 ** -23 * n0


def test_wgrad_cancellation():
    # (H~ X)^T (H~ dY) = X^T dY when both operands use the same signs along
    # the reduction (token) dimension.
    rng = np.random.default_rng(8)
    mask = workloads.rht_sign_mask()
    T = 64
    X = rng.integers(-50, 50, (T, 5)).astype(np.float32)
    dY = rng.integers(-50, 50, (T, 7)).astype(np.float32)

    def t(M):
        out = np.empty_like(M)
        for c in range(M.shape[1]):
            for b in range(T // 16):
                out[16 * b:16 * b + 16, c] = oracle.rht16(M[16 * b:16 * b + 16, c], mask)
        return out.astype(np.float64)
    np.testing.assert_array_equal(t(X).T @ t(dY), X.astype(np.float64).T @ dY.astype(np.float64))


def test_outlier_is_spread():
    # page 4 "Technologie stabilizujace ...": the transform smears outliers.
    # A lone spike of 50 in a chunk becomes 16 values of magnitude 50/4.
    x = np.zeros(16, dtype=np.float32)
    x[5] = 50.0
    y = oracle.rht16(x, workloads.rht_sign_mask())
    np.testing.assert_array_equal(np.abs(y), np.full(16, 12.5, dtype=np.float32))
    # on N(0,1) data with one x50 spike the block max/rms ratio drops
    rng = np.random.default_rng(9)
    ratios = []
    for _ in range(500):
        z = rng.standard_normal(16).astype(np.float32)
        z[rng.integers(16)] *= 50
        yz = oracle.rht16(z, 0x5A5A)
        ratios.append((np.abs(z).max() / np.sqrt(np.mean(z.astype(np.float64) ** 2)),
                       np.abs(yz).max() / np.sqrt(np.mean(yz.astype(np.float64) ** 2))))
    r = np.array(ratios)
    assert np.median(r[:, 0]) > 3.5 and np.median(r[:, 1]) < 1.6
