"""Plain CPU oracle for NanoQuant's Latent Binary ADMM (LB-ADMM).

TEST INFRASTRUCTURE. This module is the slow, obviously-correct reference
that the HIP path is checked against. Only the test-suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It shares no code with the GPU library and never imports it.

Everything runs in NumPy, float64 by default (``dtype=np.float32`` gives the
single-precision CPU throughput baseline). Library primitives serve as single
steps: matrix products, ``numpy.linalg.cholesky`` and
``scipy.linalg.solve_triangular``. Nothing is blocked, fused or reordered.

Sources (the pages are cited by title and section):
  [D]  "NANOQUANT：大语言模型的高效亚1比特量化 / NanoQuant: Efficient Sub-1-Bit
       Quantization of Large Language Models", digest at paper.rainbus.top.
       Sections used: 前置知识 (prerequisites: BPW, low-rank factorisation,
       ADMM), 研究动机 (motivation: the s1*U*V^T*s2 representation),
       核心方法 (core method: steps (a)-(c) of LB-ADMM), 方法步骤详情 (method
       steps: preconditioning, magnitude balancing, scales, sign packing),
       技术新颖性 (novelty: SVID, balancing).
  [B]  "NanoQuant的一种实现：一种灵活的二进制量化方法", blog at
       bittide.aicompass.dev, sections 什么是NanoQuant (parameter counting)
       and 待办事项 (Cholesky as the cost centre of LB-ADMM).

The pages name the steps but print no formulas for them. Where they are
silent this module takes the plainest reading that the named steps support;
each such reading is marked READING below.

Problem. Given W (m x n), positive diagonal preconditioners d_out (m) and
d_in (n), a rank r and a penalty rho, find U (m x r), V (n x r) so that the
preconditioned weight Wt = diag(d_out) W diag(d_in) is approximated by
diag(s1) sign(U) sign(V)^T diag(s2).

LB-ADMM, scaled form. The latent U is split from a binary proxy Z_U that
lives in C = { S * a b^T : S in {-1,+1}^{m x r}, a >= 0, b >= 0 } (sign
times a non-negative rank-1 magnitude), with dual Lambda_U; likewise for V.
One iteration is a U-half followed by a V-half (the V-half uses the new U):
    (a) G = V^T V + rho I,  L = chol(G),
        U = (Wt V + rho (Z_U - Lambda_U)) G^{-1}      (two triangular solves)
    (b) X = U + Lambda_U,   Z_U = SVID_T(X)
    (c) Lambda_U = X - Z_U                              (= Lambda_U + U - Z_U)
(a) minimises 1/2 ||Wt - U V^T||^2 + rho/2 ||U - Z_U + Lambda_U||^2 over U.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import scipy.linalg as sla


# ---------------------------------------------------------------------------
# a1: preconditioning  ([D] 方法步骤详情, stage 2 step (2): Wt = D_out W D_in)
# ---------------------------------------------------------------------------
def precondition(W, d_out, d_in, dtype=np.float64):
    """Wt[i, j] = d_out[i] * (W[i, j] * d_in[j]).

    READING: in float32 the two products are rounded one after the other in
    exactly this order (W times d_in first), so the float32 result is a fixed,
    reproducible function of the inputs.
    """
    W = np.asarray(W, dtype=dtype)
    d_out = np.asarray(d_out, dtype=dtype)
    d_in = np.asarray(d_in, dtype=dtype)
    t = W * d_in[None, :]
    return t * d_out[:, None]


# ---------------------------------------------------------------------------
# a2: initialisation (the pages are silent)
# ---------------------------------------------------------------------------
def init_scale(Wt, r):
    """sigma0 = (||Wt||_F^2 / (m n r))^(1/4).

    READING: U0, V0 are i.i.d. N(0, sigma0^2) so that E||U0 V0^T||_F^2 equals
    ||Wt||_F^2; rho then acts on the scale the solve actually works at.
    """
    m, n = Wt.shape
    ss = float(np.sum(np.asarray(Wt, np.float64) ** 2))
    return (ss / (m * n * r)) ** 0.25


# ---------------------------------------------------------------------------
# a7: SVID, the projection of a real matrix onto sign * rank-1 magnitude
#     ([D] 核心方法 step (b) and 技术新颖性: "Sign-Value Independent
#      Decomposition" maps the continuous latent to the binary proxy)
# ---------------------------------------------------------------------------
def svid(X, T, dtype=None):
    """Z = sign(X) * (a b^T) with (a, b) a rank-1 fit of |X|.

    READING: the rank-1 magnitude is fitted by T alternating least-squares
    (power) steps starting from b = 1:  a = |X| b / (b^T b),
    b = |X|^T a / (a^T a).  With the exact top singular pair of |X| this is
    the Euclidean projection of X onto C (for fixed a, b >= 0 the best sign is
    sign(X), and the best non-negative rank-1 fit of |X| is its top singular
    pair by Perron-Frobenius).  sign(0) = +1.  If |X| is all zero, Z = 0.
    Returns (Z, a, b).
    """
    X = np.asarray(X)
    dt = np.dtype(X.dtype if dtype is None else dtype)
    A = np.abs(X).astype(dt)
    m, r = A.shape
    a = np.zeros(m, dt)
    b = np.ones(r, dt)
    for _ in range(T):
        bb = float(b @ b)
        if bb == 0.0:
            a = np.zeros(m, dt)
            b = np.zeros(r, dt)
            break
        a = (A @ b) / dt.type(bb)
        aa = float(a @ a)
        if aa == 0.0:
            a = np.zeros(m, dt)
            b = np.zeros(r, dt)
            break
        b = (A.T @ a) / dt.type(aa)
    S = np.where(X >= 0, 1.0, -1.0).astype(dt)
    Z = S * np.outer(a, b)
    return Z.astype(dt), a.astype(dt), b.astype(dt)


def sgn(X):
    """+1 where X >= 0 (including +0 and -0), -1 elsewhere."""
    return np.where(np.asarray(X) >= 0, 1.0, -1.0)


# ---------------------------------------------------------------------------
# a3 / a4 / a5 / a6: the ridge-regularised solve through a Cholesky factor
#     ([D] 核心方法 step (a): fix V, solve the regularised linear system for
#      U by Cholesky; [B] 待办事项: Cholesky is where LB-ADMM spends its time)
# ---------------------------------------------------------------------------
def gram(V, rho):
    """G = V^T V + rho I (r x r)."""
    V = np.asarray(V)
    return V.T @ V + rho * np.eye(V.shape[1], dtype=V.dtype)


def rhs(Wt, V, Z, Lam, rho):
    """R = Wt V + rho (Z - Lambda)."""
    return Wt @ V + rho * (Z - Lam)


def cholesky(G):
    """Lower L with L L^T = G (numpy.linalg.cholesky)."""
    return np.linalg.cholesky(G)


def chol_solve(R, L):
    """U with U G = R for G = L L^T: U^T = L^-T (L^-1 R^T), two triangular solves."""
    Y = sla.solve_triangular(L, R.T, lower=True, check_finite=False)
    Ut = sla.solve_triangular(L.T, Y, lower=False, check_finite=False)
    return Ut.T


# ---------------------------------------------------------------------------
# One ADMM half-step and the full loop ([D] 核心方法 (a)-(c); [D] 前置知识,
# ADMM: x-update, z-update, dual update)
# ---------------------------------------------------------------------------
@dataclass
class State:
    U: np.ndarray
    V: np.ndarray
    Z_U: np.ndarray
    Lam_U: np.ndarray
    Z_V: np.ndarray
    Lam_V: np.ndarray
    a_U: Optional[np.ndarray] = None
    b_U: Optional[np.ndarray] = None
    a_V: Optional[np.ndarray] = None
    b_V: Optional[np.ndarray] = None

    def copy(self) -> "State":
        return State(*(None if x is None else x.copy() for x in
                       (self.U, self.V, self.Z_U, self.Lam_U, self.Z_V, self.Lam_V,
                        self.a_U, self.b_U, self.a_V, self.b_V)))


# ---------------------------------------------------------------------------
# f4: an iterative solve in place of the Cholesky factor
#     ([B] 待办事项: the author replaced the Cholesky solve of LB-ADMM by a
#      gradient-descent solver, slower than Cholesky under CUDA and faster on
#      another GPU; no details are given)
# ---------------------------------------------------------------------------
def iterative_solve(R, G, U0, steps, method="cg"):
    """Approximate U with U G = R from the warm start U0, row by row.

    READING: the sub-problem of step (a) is, for each row, the minimisation
    of 1/2 u G u^T - u r^T (G = other^T other + rho I, symmetric positive
    definite; r the row of R), whose gradient is g = u G - r. A
    gradient-descent solver takes `steps` steps per row from the factor's
    previous value:
      "gd": steepest descent with the exact step along -g:
            alpha = (g.g) / (g G g^T),  u <- u - alpha g;
      "cg": conjugate gradients (Hestenes-Stiefel): d = -g at the start, then
            alpha = (g.g) / (d G d^T),  u <- u + alpha d,  g <- g + alpha d G,
            beta = (g_new.g_new) / (g.g),  d <- -g_new + beta d.
    A row whose step denominator is not > 0 (a zero gradient) stays where it
    is. steps = 0 returns U0.
    """
    R = np.asarray(R)
    G = np.asarray(G)
    U = np.array(U0, dtype=R.dtype, copy=True)
    if method not in ("gd", "cg"):
        raise ValueError("method is 'gd' or 'cg'")
    for i in range(U.shape[0]):
        u = U[i]
        g = u @ G - R[i]
        d = -g
        gg = g @ g
        for _ in range(steps):
            if method == "gd":
                d = -g
                gg = g @ g
            Gd = d @ G
            den = d @ Gd
            if not den > 0:
                break
            alpha = gg / den
            u = u + alpha * d
            g = g + alpha * Gd
            if method == "cg":
                gg_new = g @ g
                d = -g + (gg_new / gg) * d
                gg = gg_new
        U[i] = u
    return U


def admm_half(Wt_side, other, Z, Lam, rho, T, solver=None, prev=None):
    """One half-iteration for the factor whose rows follow Wt_side's rows.

    U-half: Wt_side = Wt,   other = V.   V-half: Wt_side = Wt^T, other = U.
    Returns (new factor, Z, Lambda, a, b).
    READINGS: the solve uses the latent of the other factor (not its proxy);
    the dual is the scaled dual with unit step; SVID acts on X = new + Lambda.
    solver = (method, steps) replaces the Cholesky solve by iterative_solve
    warm-started from `prev`, the factor's value before this half.
    """
    G = gram(other, rho)
    R = rhs(Wt_side, other, Z, Lam, rho)
    if solver is None:
        F = chol_solve(R, cholesky(G))
    else:
        F = iterative_solve(R, G, prev, solver[1], solver[0])
    X = F + Lam
    Znew, a, b = svid(X, T)
    Lnew = X - Znew
    return F, Znew, Lnew, a, b


def init_state(Wt, r, T, EU=None, EV=None, U0=None, V0=None, dtype=np.float64):
    """Initial ADMM state: U0, V0, Lambda = 0, Z = SVID_T(U0), SVID_T(V0).

    Either pass the standard-normal draws EU, EV (scaled here by sigma0) or the
    exact starting latents U0, V0 (warm start / planted tests).
    """
    Wt = np.asarray(Wt, dtype)
    if U0 is None:
        s0 = init_scale(Wt, r)
        U0 = s0 * np.asarray(EU, dtype)
        V0 = s0 * np.asarray(EV, dtype)
    U0 = np.asarray(U0, dtype).copy()
    V0 = np.asarray(V0, dtype).copy()
    Z_U, aU, bU = svid(U0, T)
    Z_V, aV, bV = svid(V0, T)
    return State(U0, V0, Z_U, np.zeros_like(U0), Z_V, np.zeros_like(V0), aU, bU, aV, bV)


def iterate(Wt, st: State, rho, T, iters, dtype=np.float64, solver=None) -> State:
    """Run ``iters`` full iterations (U-half, then V-half) from ``st``;
    ``solver`` as in admm_half (None: Cholesky)."""
    Wt = np.asarray(Wt, dtype)
    WtT = Wt.T
    st = st.copy()
    for _ in range(iters):
        st.U, st.Z_U, st.Lam_U, st.a_U, st.b_U = admm_half(Wt, st.V, st.Z_U, st.Lam_U, rho, T,
                                                           solver, st.U)
        st.V, st.Z_V, st.Lam_V, st.a_V, st.b_V = admm_half(WtT, st.U, st.Z_V, st.Lam_V, rho, T,
                                                           solver, st.V)
    return st


# ---------------------------------------------------------------------------
# a8 / a9 / a10: magnitude balancing, scales, sign packing
#     ([D] 方法步骤详情 stage 2 step (2): after convergence, balance the
#      magnitudes to remove the scale ambiguity, then extract channel scales
#      s1 and s2; step (3): take signs and pack them to an integer format;
#      [D] 研究动机: the representation W ~ s1 U_{+-1} V_{+-1}^T s2)
# ---------------------------------------------------------------------------
def balance(U, V):
    """Per rank column k: c = sqrt(||v_k|| / ||u_k||), u_k *= c, v_k /= c.

    U V^T is unchanged and afterwards ||u_k|| = ||v_k||.
    READING: a column where either norm is zero is left as is.
    """
    U = np.array(U, copy=True)
    V = np.array(V, copy=True)
    nu = np.sqrt(np.sum(U * U, axis=0))
    nv = np.sqrt(np.sum(V * V, axis=0))
    ok = (nu > 0) & (nv > 0)
    c = np.ones_like(nu)
    c[ok] = np.sqrt(nv[ok] / nu[ok])
    return U * c[None, :], V / c[None, :], c


def row_scales(F):
    """s_i = mean_k |F[i, k]|: the least-squares scalar for F[i, :] ~ s * sign(F[i, :])."""
    return np.mean(np.abs(F), axis=1)


def pack_signs(X):
    """Bits of sign(X) along each row: bit = [x >= 0], LSB-first in uint32 words.

    Word w of row i holds columns 32 w .. 32 w + 31, column 32 w + k in bit k;
    the tail of the last word is zero.  Returns uint32 (rows, ceil(cols/32)).
    """
    X = np.asarray(X)
    rows, cols = X.shape
    nw = (cols + 31) // 32
    out = np.zeros((rows, nw), np.uint64)
    pos = X >= 0
    for j in range(cols):
        out[:, j // 32] |= pos[:, j].astype(np.uint64) << np.uint64(j % 32)
    return out.astype(np.uint32)


def unpack_signs(bits, cols):
    """Inverse of pack_signs: +1 / -1 float64 matrix (rows, cols)."""
    bits = np.asarray(bits, np.uint32)
    rows = bits.shape[0]
    S = np.empty((rows, cols))
    for j in range(cols):
        bit = (bits[:, j // 32] >> np.uint32(j % 32)) & np.uint32(1)
        S[:, j] = np.where(bit == 1, 1.0, -1.0)
    return S


# ---------------------------------------------------------------------------
# a11: reconstruction error and bits per weight
#     ([D] 前置知识 BPW; [D] 研究动机; [B] 什么是NanoQuant, parameter count)
# ---------------------------------------------------------------------------
def reconstruct(s1, SU, SV, s2):
    """diag(s1) SU SV^T diag(s2)."""
    return (s1[:, None] * (SU @ SV.T)) * s2[None, :]


def rel_error(target, s1, SU, SV, s2):
    """||target - diag(s1) SU SV^T diag(s2)||_F / ||target||_F (dense, in float64)."""
    target = np.asarray(target, np.float64)
    E = reconstruct(np.asarray(s1, np.float64), np.asarray(SU, np.float64),
                    np.asarray(SV, np.float64), np.asarray(s2, np.float64))
    return float(np.linalg.norm(target - E) / np.linalg.norm(target))


def bpw(m, n, r, scale_bits=0):
    """Bits per weight: r (m + n) sign bits plus scale_bits per entry of s1, s2, over m n."""
    return (r * (m + n) + scale_bits * (m + n)) / (m * n)


# ---------------------------------------------------------------------------
# The whole per-layer path
# ---------------------------------------------------------------------------
@dataclass
class Result:
    U: np.ndarray          # balanced latent U (m x r)
    V: np.ndarray          # balanced latent V (n x r)
    s1: np.ndarray         # stored scale, W space: s1_wt / d_out
    s2: np.ndarray         # stored scale, W space: s2_wt / d_in
    s1_wt: np.ndarray      # scale in preconditioned space
    s2_wt: np.ndarray
    U_bits: np.ndarray     # uint32 (m, ceil(r/32))
    V_bits: np.ndarray     # uint32 (n, ceil(r/32))
    rel_err_wt: float      # error in Wt space
    rel_err_w: float       # error in W space
    bpw: float             # sign bits only
    bpw_fp16_scales: float
    state: State           # unbalanced ADMM state after the last iteration
    sigma0: float


def finish(Wt, W, d_out, d_in, U, V, compute_error=True):
    """Balance, scales, signs, packing and errors from the final latent U, V.

    READINGS: the final signs are those of the balanced latent; the scales are
    the row means of |balanced latent|; the stored scales fold the
    preconditioners back out (s1 / d_out, s2 / d_in) so that
    W ~ diag(s1 / d_out) sign(U) sign(V)^T diag(s2 / d_in).
    """
    Ub, Vb, _ = balance(U, V)
    s1w = row_scales(Ub)
    s2w = row_scales(Vb)
    SU = sgn(Ub)
    SV = sgn(Vb)
    d_out = np.asarray(d_out, np.float64)
    d_in = np.asarray(d_in, np.float64)
    s1 = s1w / d_out
    s2 = s2w / d_in
    e_wt = e_w = float("nan")
    if compute_error:
        e_wt = rel_error(Wt, s1w, SU, SV, s2w)
        e_w = rel_error(W, s1, SU, SV, s2)
    return Ub, Vb, s1, s2, s1w, s2w, pack_signs(Ub), pack_signs(Vb), e_wt, e_w


def lbadmm(W, d_out, d_in, r, rho=1.0, iters=20, svid_steps=5, EU=None, EV=None,
           U0=None, V0=None, dtype=np.float64, compute_error=True) -> Result:
    """Full per-layer LB-ADMM: precondition, init, iterate, finish."""
    W = np.asarray(W)
    m, n = W.shape
    Wt = precondition(W, d_out, d_in, dtype)
    s0 = init_scale(Wt, r)
    st = init_state(Wt, r, svid_steps, EU=EU, EV=EV, U0=U0, V0=V0, dtype=dtype)
    st = iterate(Wt, st, rho, svid_steps, iters, dtype)
    Ub, Vb, s1, s2, s1w, s2w, ub, vb, e_wt, e_w = finish(
        Wt, np.asarray(W, np.float64), d_out, d_in, st.U, st.V, compute_error)
    return Result(Ub, Vb, s1, s2, s1w, s2w, ub, vb, e_wt, e_w,
                  bpw(m, n, r), bpw(m, n, r, 16), st, s0)


def objective(Wt, U, V, Z_U, Lam_U, Z_V, Lam_V, rho):
    """Scaled augmented Lagrangian, up to the constant dual terms:
    1/2||Wt - U V^T||^2 + rho/2 ||U - Z_U + Lam_U||^2 + rho/2 ||V - Z_V + Lam_V||^2."""
    return (0.5 * np.sum((Wt - U @ V.T) ** 2)
            + 0.5 * rho * np.sum((U - Z_U + Lam_U) ** 2)
            + 0.5 * rho * np.sum((V - Z_V + Lam_V) ** 2))
