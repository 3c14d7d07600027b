"""Plain CPU oracle for the STE refinement of one factorised layer.

TEST INFRASTRUCTURE. Only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code with
the GPU library and never imports it. NumPy, float64.

Sources (cited by title and section):
  [D] "NANOQUANT：大语言模型的高效亚1比特量化", digest at paper.rainbus.top:
      section 方法步骤详情, stage 2 step (3) (component refinement): the
      continuous latents U, V and the scales s1, s2 are optimised jointly
      with a straight-through estimator (STE) to minimise the MSE between
      the quantised and the full-precision outputs; afterwards the signs are
      taken and packed. Section 复现评估 (reproduction): learning rate 1e-4
      to 1e-6, batch size 1-4, 8 epochs, cosine learning-rate schedule.

READINGS (the pages give no formulas):
  - One linear layer stands in for the block: the full-precision output of
    a batch of activations X (tokens x n) is Y = X W^T, the quantised one
    Yq = X Wq^T with Wq = diag(s1) sign(U) sign(V)^T diag(s2) (the W-space
    scales the factorisation returns). The loss is the mean over the batch's
    tokens x m outputs of (Yq - Y)^2.
  - sign(x) = +1 for x >= 0, -1 otherwise (as for the packed bits). The STE
    passes the gradient through sign unchanged: dL/dU = dL/dsign(U).
  - The optimiser is Adam (PyTorch's form: beta1 0.9, beta2 0.999,
    eps 1e-8, bias-corrected moments, no weight decay), one optimiser over
    U, V, s1, s2; the pages name the learning rates, not the optimiser.
  - The cosine schedule runs from lr_max at the first step to lr_min after
    the last: lr_t = lr_min + (lr_max - lr_min) (1 + cos(pi t / K)) / 2 for
    steps t = 0 .. K-1 of K.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def sgn(X):
    return np.where(np.asarray(X) >= 0, 1.0, -1.0)


def forward(X, U, V, s1, s2):
    """Yq = X Wq^T, right to left: ((X diag(s2)) S_V) S_U^T diag(s1)."""
    A = np.asarray(X, np.float64) * np.asarray(s2, np.float64)[None, :]
    P = A @ sgn(V)
    Q = P @ sgn(U).T
    return Q * np.asarray(s1, np.float64)[None, :]


def loss(X, Y, U, V, s1, s2):
    """Mean of (Yq - Y)^2 over the batch's tokens x outputs."""
    E = forward(X, U, V, s1, s2) - np.asarray(Y, np.float64)
    return float(np.mean(E * E))


def grads(X, Y, U, V, s1, s2):
    """(dU, dV, ds1, ds2) of the loss, sign passed straight through.

    With A = X diag(s2), P = A S_V, Q = P S_U^T, Yq = Q diag(s1) and
    G = dL/dYq = 2 (Yq - Y) / (T m):
      ds1_i = sum_t G_ti Q_ti;   dQ = G diag(s1);
      dS_U = dQ^T P;             dP = dQ S_U;
      dS_V = A^T dP;             dA = dP S_V^T;   ds2_j = sum_t dA_tj X_tj.
    """
    X = np.asarray(X, np.float64)
    s1 = np.asarray(s1, np.float64)
    s2 = np.asarray(s2, np.float64)
    SU, SV = sgn(U), sgn(V)
    A = X * s2[None, :]
    P = A @ SV
    Q = P @ SU.T
    E = Q * s1[None, :] - np.asarray(Y, np.float64)
    G = 2.0 * E / E.size
    ds1 = np.sum(G * Q, axis=0)
    dQ = G * s1[None, :]
    dU = dQ.T @ P
    dP = dQ @ SU
    dV = A.T @ dP
    dA = dP @ SV.T
    ds2 = np.sum(dA * X, axis=0)
    return dU, dV, ds1, ds2


def cosine_lr(t, K, lr_max=1e-4, lr_min=1e-6):
    """Learning rate of step t (0-based) of K."""
    return lr_min + (lr_max - lr_min) * (1.0 + np.cos(np.pi * t / K)) / 2.0


@dataclass
class AdamState:
    m: list
    v: list
    t: int = 0


def adam_init(params):
    return AdamState([np.zeros_like(p, dtype=np.float64) for p in params],
                     [np.zeros_like(p, dtype=np.float64) for p in params], 0)


def adam_step(params, gs, st: AdamState, lr, b1=0.9, b2=0.999, eps=1e-8):
    """One Adam update of every parameter (returns new arrays)."""
    st.t += 1
    out = []
    for k, (p, g) in enumerate(zip(params, gs)):
        st.m[k] = b1 * st.m[k] + (1.0 - b1) * g
        st.v[k] = b2 * st.v[k] + (1.0 - b2) * g * g
        mh = st.m[k] / (1.0 - b1 ** st.t)
        vh = st.v[k] / (1.0 - b2 ** st.t)
        out.append(p - lr * mh / (np.sqrt(vh) + eps))
    return out


def refine(X, Y, U, V, s1, s2, batches, lr_max=1e-4, lr_min=1e-6):
    """STE refinement over `batches` (a list of token-index arrays, one per
    step, epochs already laid out). Returns (U, V, s1, s2, losses) with the
    loss of each step's batch before its update."""
    params = [np.asarray(p, np.float64).copy() for p in (U, V, s1, s2)]
    st = adam_init(params)
    K = len(batches)
    losses = []
    for t, idx in enumerate(batches):
        Xb, Yb = X[idx], Y[idx]
        losses.append(loss(Xb, Yb, *params))
        gs = grads(Xb, Yb, *params)
        params = adam_step(params, gs, st, cosine_lr(t, K, lr_max, lr_min))
    return params[0], params[1], params[2], params[3], losses
