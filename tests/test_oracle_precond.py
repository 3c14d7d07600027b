"""Pins of oracle/precond.py (the Ledoit-Wolf diagonal preconditioners of the
calibration stage) to things other than itself: scikit-learn's
ledoit_wolf (an independent implementation of the same estimator), closed
forms, invariances, and the diagonal K-FAC identity behind the square root."""
import numpy as np
import pytest
from sklearn.covariance import ledoit_wolf as sk_ledoit_wolf

from oracle import precond as P


def _acts(seed, N, p, outliers=0.0):
    rng = np.random.default_rng(seed)
    scale = rng.lognormal(0.0, 1.0, p)
    if outliers:
        k = max(1, int(outliers * p))
        scale[rng.choice(p, k, replace=False)] *= 20.0
    mean = 0.3 * rng.standard_normal(p) * scale
    return mean + rng.standard_normal((N, p)) * scale


@pytest.mark.parametrize("N, p, out", [(50, 8, 0.0), (7, 20, 0.0), (200, 33, 0.05), (3, 3, 0.0),
                                       (400, 64, 0.02)])
def test_matches_scikit_learn_ledoit_wolf(N, p, out):
    # sklearn with assume_centered=True is the same estimator on the
    # uncentered second moment, computed its own way (block sums of X^2)
    Z = _acts(N + p, N, p, out)
    sig, shrink, m = P.ledoit_wolf(Z)
    sk_sig, sk_shrink = sk_ledoit_wolf(Z, assume_centered=True)
    assert shrink == pytest.approx(sk_shrink, rel=1e-10, abs=1e-14)
    np.testing.assert_allclose(sig, sk_sig, rtol=1e-10, atol=1e-12 * np.abs(sk_sig).max())
    d, s2 = P.diag_preconditioner(Z)
    np.testing.assert_allclose(d, np.sqrt(np.diag(sk_sig)), rtol=1e-10)
    assert s2 == shrink


def test_second_moment_is_uncentered():
    Z = _acts(1, 30, 5)
    S = P.second_moment(Z)
    np.testing.assert_allclose(S, sum(np.outer(z, z) for z in Z) / 30, rtol=1e-13)
    assert not np.allclose(S, np.cov(Z.T, bias=True))


def test_isotropic_and_single_sample_need_no_shrinkage():
    # columns orthogonal with equal norms: S = c^2 I = m I, so every
    # shrinkage gives the same Sigma* (d2 is zero up to rounding) and d = c
    Q, _ = np.linalg.qr(np.random.default_rng(2).standard_normal((40, 6)))
    Z = 3.0 * np.sqrt(40) * Q
    d, shrink = P.diag_preconditioner(Z)
    assert 0.0 <= shrink <= 1.0
    np.testing.assert_allclose(d, 3.0, rtol=1e-12)
    # one sample: z z^T - S = 0, so b2bar = 0 and d = |z|
    z = np.array([[1.0, -2.0, 0.5, 4.0]])
    d, shrink = P.diag_preconditioner(z)
    assert shrink == 0.0
    np.testing.assert_allclose(d, np.abs(z[0]), rtol=1e-15)


def test_invariances_and_bounds():
    Z = _acts(3, 120, 24, 0.05)
    d, shrink = P.diag_preconditioner(Z)
    assert 0.0 <= shrink <= 1.0
    # scaling the sample scales d, not the shrinkage
    d2, shrink2 = P.diag_preconditioner(-2.5 * Z)
    assert shrink2 == pytest.approx(shrink, rel=1e-12)
    np.testing.assert_allclose(d2, 2.5 * d, rtol=1e-12)
    # permuting features permutes d; permuting tokens changes nothing
    perm = np.random.default_rng(4).permutation(24)
    np.testing.assert_allclose(P.diag_preconditioner(Z[:, perm])[0], d[perm], rtol=1e-12)
    tok = np.random.default_rng(5).permutation(120)
    np.testing.assert_allclose(P.diag_preconditioner(Z[tok])[0], d, rtol=1e-12)
    # d^2 is the convex combination of S_jj and m
    S = P.second_moment(Z)
    m = np.trace(S) / 24
    np.testing.assert_allclose(d ** 2, (1 - shrink) * np.diag(S) + shrink * m, rtol=1e-12)
    lo = np.minimum(np.diag(S), m)
    hi = np.maximum(np.diag(S), m)
    assert np.all(d ** 2 >= lo * (1 - 1e-12)) and np.all(d ** 2 <= hi * (1 + 1e-12))


def test_diagonal_kfac_weighting_is_the_preconditioned_error():
    # sum_ij Sout_ii Sin_jj E_ij^2 == ||D_out E D_in||_F^2 with D = sqrt(diag)
    rng = np.random.default_rng(6)
    X_in = _acts(7, 90, 12)
    Z_out = _acts(8, 90, 9)
    d_out, d_in = P.preconditioners(X_in, Z_out)
    s_in = np.diag(P.ledoit_wolf(X_in)[0])
    s_out = np.diag(P.ledoit_wolf(Z_out)[0])
    E = rng.standard_normal((9, 12))
    lhs = np.sum(s_out[:, None] * s_in[None, :] * E ** 2)
    rhs = np.linalg.norm(np.diag(d_out) @ E @ np.diag(d_in)) ** 2
    assert lhs == pytest.approx(rhs, rel=1e-12)
