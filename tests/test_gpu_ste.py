"""GPU parity of the STE refinement (nq_ste_*) against oracle/ste.py on the
same seeded layer, activations and batches.

The GPU runs the products in fp32 on the matrix cores (the signs are exact),
the oracle in fp64. The loss of every step is held to 1e-5 relative. One
Adam step moves a parameter by -lr m^/(sqrt(v^) + eps), a bounded function
of the gradient, so parameters are held to 1e-6 relative plus 1e-3 lr
absolute (the update agrees to a part in a thousand; a sign that differs
between the two gradients at rounding level would cost 2 lr and fail it).
At 4096 x 4096, r = 2048 with the bench's 8192-token batches, the loss and
sampled rows of U (with s1) after one step are compared.
"""
import numpy as np
import pytest

from oracle import ste as S
from synth import make_activations

pytestmark = pytest.mark.gpu


def T(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def H(t):
    return t.detach().cpu().numpy()


def layer(seed, m, n, r, N):
    rng = np.random.default_rng(seed)
    W = (0.02 * rng.standard_normal((m, n))).astype(np.float32)
    X = make_activations(N, n, seed + 1)
    Y = (X.astype(np.float64) @ W.T.astype(np.float64)).astype(np.float32)
    U = (0.1 * rng.standard_normal((m, r))).astype(np.float32)
    V = (0.1 * rng.standard_normal((n, r))).astype(np.float32)
    s1 = rng.uniform(0.005, 0.03, m).astype(np.float32)
    s2 = rng.uniform(0.005, 0.03, n).astype(np.float32)
    return X, Y, U, V, s1, s2


@pytest.mark.parametrize("m, n, r, N, bt, steps", [(300, 260, 70, 600, 200, 4),
                                                   (256, 512, 128, 1024, 512, 3),
                                                   (64, 48, 8, 100, 37, 5),
                                                   (520, 300, 96, 700, 700, 2)])
def test_ste_steps_match_oracle(gpu, m, n, r, N, bt, steps):
    import torch
    import sub_bit_weight_lb_amd as nq
    X, Y, U, V, s1, s2 = layer(m + n, m, n, r, N)
    rng = np.random.default_rng(3)
    batches = [rng.permutation(N)[:bt].astype(np.int32) for _ in range(steps)]
    print(f"case {m}x{n} r={r} N={N} batch={bt} steps={steps}", flush=True)
    with nq.STERefiner(m, n, r, bt) as h:
        h.set_params(T(U, gpu), T(V, gpu), T(s1, gpu), T(s2, gpu))
        losses = h.refine(T(X, gpu), T(Y, gpu), [T(b, gpu) for b in batches])
        Ug, Vg, ag, bg = (H(x) for x in h.params())
    Uo, Vo, ao, bo, lo = S.refine(X.astype(np.float64), Y.astype(np.float64), U, V, s1, s2,
                                  [b.astype(np.int64) for b in batches])
    np.testing.assert_allclose(losses, lo, rtol=1e-5)
    lr = 1e-4
    for name, g, o in (("U", Ug, Uo), ("V", Vg, Vo), ("s1", ag, ao), ("s2", bg, bo)):
        np.testing.assert_allclose(g, o, rtol=1e-6, atol=1e-3 * lr, err_msg=name)
    # something moved: every step moves every parameter with a nonzero gradient
    assert np.abs(Ug - U).max() > 0.5 * lr and np.abs(ag - s1).max() > 0.5 * lr


def test_ste_contiguous_rows_and_errors(gpu):
    import sub_bit_weight_lb_amd as nq
    m, n, r, N = 128, 96, 32, 300
    X, Y, U, V, s1, s2 = layer(7, m, n, r, N)
    with nq.STERefiner(m, n, r, N) as h:
        with pytest.raises(nq.NQError):
            h.step(T(X, gpu), T(Y, gpu), 1e-4)              # no parameters yet
        h.set_params(T(U, gpu), T(V, gpu), T(s1, gpu), T(s2, gpu))
        h.step(T(X, gpu), T(Y, gpu), 1e-4)                   # rows = None: all N rows
        l0 = h.last_loss()
        with pytest.raises(ValueError):
            h.step(T(X[:, :n - 1], gpu), T(Y, gpu), 1e-4)
    assert l0 == pytest.approx(S.loss(X, Y, U, V, s1, s2), rel=1e-5)
    with pytest.raises(nq.NQError):
        nq.STERefiner(0, 5, 5, 5)
    with pytest.raises(nq.NQError):
        nq.STERefiner(5, 5, (1 << 13) + 1, 5)


def test_ste_full_size_one_step(gpu):
    import sub_bit_weight_lb_amd as nq
    m = n = 4096
    r, Tn = 2048, 8192
    X, Y, U, V, s1, s2 = layer(11, m, n, r, Tn)
    print(f"case {m}x{n} r={r} T={Tn}", flush=True)
    with nq.STERefiner(m, n, r, Tn) as h:
        h.set_params(T(U, gpu), T(V, gpu), T(s1, gpu), T(s2, gpu))
        h.step(T(X, gpu), T(Y, gpu), 1e-4)
        loss = h.last_loss()
        Ug, _, ag, _ = (H(x) for x in h.params())
    # oracle pieces in fp64: the loss, and rows of dU / entries of ds1
    X64 = X.astype(np.float64)
    A = X64 * s2.astype(np.float64)
    P = A @ S.sgn(V)
    SU = S.sgn(U)
    Q = P @ SU.T
    E = Q * s1.astype(np.float64) - Y
    lo = float(np.mean(E * E))
    print(f"  loss gpu {loss:.9e} oracle {lo:.9e}", flush=True)
    assert loss == pytest.approx(lo, rel=1e-5)
    G = 2.0 * E / E.size
    rows = np.random.default_rng(2).choice(m, 8, replace=False)
    for i in rows:
        dQi = G[:, i] * s1[i]
        dUi = dQi @ P
        ds1i = float(np.sum(G[:, i] * Q[:, i]))
        # first Adam step: m^ = g, v^ = g^2
        np.testing.assert_allclose(Ug[i], U[i] - 1e-4 * dUi / (np.abs(dUi) + 1e-8),
                                   rtol=1e-6, atol=1e-7)
        assert ag[i] == pytest.approx(s1[i] - 1e-4 * ds1i / (abs(ds1i) + 1e-8), rel=1e-6, abs=1e-7)
