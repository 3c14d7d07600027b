"""Plain CPU oracle for the diagonal preconditioners of NanoQuant's first
stage (global calibration).

TEST INFRASTRUCTURE. Only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code with
the GPU library and never imports it. NumPy, float64.

Sources (cited by title and section):
  [D] "NANOQUANT：大语言模型的高效亚1比特量化", digest at paper.rainbus.top:
      section 方法步骤详情, stage 1: calibration samples are run forward,
      statistics z_in and z_out of every linear layer's activations are
      collected, and robust diagonal preconditioners D_in and D_out are built
      from them with Ledoit-Wolf shrinkage; section 前置知识 (K-FAC): the
      method uses a simplified diagonal K-FAC preconditioner for a
      Hessian-aware reconstruction objective.
  [LW] O. Ledoit, M. Wolf, "A well-conditioned estimator for
      large-dimensional covariance matrices", J. Multivariate Analysis 88
      (2004): the shrinkage estimator and its sample quantities m, d^2, b^2.

The pages give no formula. READINGS, the plainest ones the passages support:
  - z_in (z_out) is a sample matrix Z, N tokens x p features, of the layer's
    input (output) side. The statistic is the uncentered second moment
    S = Z^T Z / N, as in K-FAC's Kronecker factors (E[x x^T]): a feature's
    mean is part of its weight in the reconstruction error, so it is not
    removed.
  - Ledoit-Wolf shrinks S toward m I with the intensity of [LW], written
    with the normalised Frobenius norm ||A||^2 = tr(A A^T) / p:
        m  = tr(S) / p
        d2 = ||S - m I||^2
        b2bar = (1 / N^2) sum_k ||z_k z_k^T - S||^2
        b2 = min(b2bar, d2),  shrinkage = b2 / d2  (0 when d2 = 0)
        Sigma* = shrinkage m I + (1 - shrinkage) S.
  - The preconditioner is D = diag(Sigma*)^(1/2): with a diagonal K-FAC
    weighting the reconstruction error sum_ij Sigma*_out,ii Sigma*_in,jj
    (W - W^)_ij^2 is ||D_out (W - W^) D_in||_F^2, which is the preconditioned
    target D_out W D_in of stage 2.
"""
from __future__ import annotations

import numpy as np


def second_moment(Z):
    """S = Z^T Z / N (p x p), float64."""
    Z = np.asarray(Z, np.float64)
    return Z.T @ Z / Z.shape[0]


def ledoit_wolf(Z):
    """(Sigma*, shrinkage, m) for the sample Z (N x p), per [LW] with the
    uncentered second moment; b2bar by its definition, a sum over samples."""
    Z = np.asarray(Z, np.float64)
    N, p = Z.shape
    S = second_moment(Z)
    m = np.trace(S) / p
    I = np.eye(p)
    d2 = np.sum((S - m * I) ** 2) / p
    b2bar = 0.0
    for k in range(N):
        zk = Z[k][:, None]
        b2bar += np.sum((zk @ zk.T - S) ** 2) / p
    b2bar /= N * N
    b2 = min(b2bar, d2)
    shrink = 0.0 if d2 == 0.0 else b2 / d2
    return shrink * m * I + (1.0 - shrink) * S, shrink, m


def diag_preconditioner(Z):
    """(d, shrinkage): d = sqrt(diag(Sigma*)) for the sample Z (N x p)."""
    sig, shrink, _ = ledoit_wolf(Z)
    return np.sqrt(np.diag(sig)), shrink


def preconditioners(X_in, Z_out):
    """(d_out, d_in) for a layer from its input-side sample X_in (N x n) and
    output-side sample Z_out (N x m): the diagonals of D_out and D_in."""
    d_in, _ = diag_preconditioner(X_in)
    d_out, _ = diag_preconditioner(Z_out)
    return d_out, d_in
