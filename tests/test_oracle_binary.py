"""Pins for oracle.binary (the product with a low-rank binary layer).

- the dense route: X W^T with W formed by oracle.lbadmm.reconstruct (a
  different association order) on shapes with m != n and r not a multiple
  of 32;
- brute force: the double sum over k and j written out for tiny shapes;
- a closed form: with S_U = S_V = H, a Sylvester-Hadamard matrix (H H^T =
  r I), W = r diag(s1 s2), so y = r s1 s2 x.
"""
import numpy as np
import pytest

from oracle import binary as OB
from oracle import lbadmm as O


def _layer(rng, m, n, r):
    SU = np.where(rng.random((m, r)) < 0.5, -1.0, 1.0)
    SV = np.where(rng.random((n, r)) < 0.5, -1.0, 1.0)
    s1 = rng.uniform(0.1, 2.0, m)
    s2 = rng.uniform(0.1, 2.0, n)
    return SU, SV, s1, s2


@pytest.mark.parametrize("m,n,r,B", [(7, 5, 3, 1), (40, 70, 33, 4), (96, 64, 64, 2), (130, 17, 95, 3)])
def test_matches_dense_product(m, n, r, B):
    rng = np.random.default_rng(m * 31 + n + r)
    SU, SV, s1, s2 = _layer(rng, m, n, r)
    X = rng.standard_normal((B, n))
    Y = OB.binary_matmul(X, O.pack_signs(SU), O.pack_signs(SV), r, s1, s2)
    W = O.reconstruct(s1, SU, SV, s2)
    assert Y.shape == (B, m)
    np.testing.assert_allclose(Y, X @ W.T, rtol=1e-12, atol=1e-12 * np.abs(X @ W.T).max())


@pytest.mark.parametrize("m,n,r,B", [(3, 4, 2, 1), (5, 2, 7, 2), (4, 6, 33, 1)])
def test_brute_force_sum(m, n, r, B):
    rng = np.random.default_rng(100 + m + n + r)
    SU, SV, s1, s2 = _layer(rng, m, n, r)
    X = rng.standard_normal((B, n))
    Y = OB.binary_matmul(X, O.pack_signs(SU), O.pack_signs(SV), r, s1, s2)
    for b in range(B):
        for i in range(m):
            acc = 0.0
            for k in range(r):
                for j in range(n):
                    acc += s1[i] * SU[i, k] * SV[j, k] * s2[j] * X[b, j]
            assert abs(Y[b, i] - acc) <= 1e-12 * max(1.0, abs(acc))


def _hadamard(r):
    H = np.ones((1, 1))
    while H.shape[0] < r:
        H = np.block([[H, H], [H, -H]])
    return H


@pytest.mark.parametrize("r", [1, 2, 8, 64])
def test_hadamard_closed_form(r):
    rng = np.random.default_rng(r)
    H = _hadamard(r)
    assert np.array_equal(H @ H.T, r * np.eye(r))
    s1 = rng.uniform(0.5, 1.5, r)
    s2 = rng.uniform(0.5, 1.5, r)
    X = rng.standard_normal((3, r))
    Y = OB.binary_matmul(X, O.pack_signs(H), O.pack_signs(H), r, s1, s2)
    np.testing.assert_allclose(Y, r * s1[None, :] * s2[None, :] * X, rtol=1e-12, atol=1e-12)


def test_single_vector_input():
    rng = np.random.default_rng(9)
    SU, SV, s1, s2 = _layer(rng, 6, 9, 5)
    x = rng.standard_normal(9)
    Y = OB.binary_matmul(x, O.pack_signs(SU), O.pack_signs(SV), 5, s1, s2)
    assert Y.shape == (1, 6)
    np.testing.assert_allclose(Y[0], O.reconstruct(s1, SU, SV, s2) @ x, rtol=1e-12, atol=1e-12)
