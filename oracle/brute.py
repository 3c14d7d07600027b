"""Exhaustive search for tiny low-rank binary factorisations (test infrastructure).

For m, n <= 4 and r <= 2 every pair of sign matrices SU in {-1,+1}^{m x r},
SV in {-1,+1}^{n x r} is enumerated (at most 2^16 pairs). For each pair the
row/column scales are fitted by alternating least squares on
    f(s1, s2) = || T - diag(s1) P diag(s2) ||_F^2,   P = SU SV^T,
from several starts. The smallest value found bounds from above the best
objective any method reaching the representation diag(s1) SU SV^T diag(s2)
([D] 研究动机: W ~ s1 U_{+-1} V_{+-1}^T s2) can attain on T, and a method's
own objective can never fall below the true minimum.

Only the test-suite imports this module.
"""
from __future__ import annotations

import itertools

import numpy as np


def _sign_matrices(rows, r):
    """All {-1,+1}^{rows x r} matrices, shape (2^(rows r), rows, r)."""
    k = rows * r
    codes = np.arange(2 ** k, dtype=np.int64)
    bits = (codes[:, None] >> np.arange(k)[None, :]) & 1
    return (2.0 * bits - 1.0).reshape(-1, rows, r)


def fit_scales(T, P, s1, s2, sweeps=200):
    """ALS on s1, s2 for fixed P (batched over the leading axis). Returns (f, s1, s2)."""
    for _ in range(sweeps):
        # d f / d s1_i = 0  ->  s1_i = sum_j T_ij P_ij s2_j / sum_j P_ij^2 s2_j^2
        num = np.einsum("ij,bij,bj->bi", T, P, s2)
        den = np.einsum("bij,bj->bi", P * P, s2 * s2)
        s1 = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)
        num = np.einsum("ij,bij,bi->bj", T, P, s1)
        den = np.einsum("bij,bi->bj", P * P, s1 * s1)
        s2 = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)
    E = T[None] - s1[:, :, None] * P * s2[:, None, :]
    return np.sum(E * E, axis=(1, 2)), s1, s2


def brute_force_min(T, r, starts=4, seed=0):
    """Smallest ||T - diag(s1) SU SV^T diag(s2)||_F^2 found over all sign pairs.

    Returns (f_min, SU, SV, s1, s2) of the best pair.
    """
    T = np.asarray(T, np.float64)
    m, n = T.shape
    assert m <= 4 and n <= 4 and r <= 2, "exhaustive search is for tiny shapes only"
    SUs = _sign_matrices(m, r)
    SVs = _sign_matrices(n, r)
    rng = np.random.default_rng(seed)
    best = (np.inf, None, None, None, None)
    for iu in range(len(SUs)):
        P = np.einsum("ik,bjk->bij", SUs[iu], SVs)          # (nV, m, n)
        for s in range(starts):
            if s == 0:
                s1 = np.ones((len(SVs), m))
                s2 = np.ones((len(SVs), n))
            else:
                s1 = rng.uniform(0.1, 2.0, (len(SVs), m))
                s2 = rng.uniform(0.1, 2.0, (len(SVs), n))
            f, a, b = fit_scales(T, P, s1, s2)
            k = int(np.argmin(f))
            if f[k] < best[0]:
                best = (float(f[k]), SUs[iu].copy(), SVs[k].copy(), a[k].copy(), b[k].copy())
    return best


def objective(T, s1, SU, SV, s2):
    """||T - diag(s1) SU SV^T diag(s2)||_F^2 written out entry by entry."""
    T = np.asarray(T, np.float64)
    m, n = T.shape
    r = SU.shape[1]
    f = 0.0
    for i, j in itertools.product(range(m), range(n)):
        p = sum(SU[i, k] * SV[j, k] for k in range(r))
        e = T[i, j] - s1[i] * p * s2[j]
        f += e * e
    return f
