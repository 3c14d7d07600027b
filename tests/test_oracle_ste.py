"""Pins of oracle/ste.py (STE refinement of a factorised layer) to things
other than itself: the dense layer product, finite differences of the loss,
PyTorch's Adam and cosine schedule (independent implementations of the
same optimiser and schedule), a hand-worked Adam case, and planted cases."""
import numpy as np
import pytest
import torch

from oracle import ste as S


def _layer(seed, T=40, m=9, n=11, r=4):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, n))
    W = 0.3 * rng.standard_normal((m, n))
    U = rng.standard_normal((m, r))
    V = rng.standard_normal((n, r))
    s1 = rng.uniform(0.2, 1.0, m)
    s2 = rng.uniform(0.2, 1.0, n)
    return X, X @ W.T, U, V, s1, s2


def test_forward_is_the_dense_layer():
    X, Y, U, V, s1, s2 = _layer(1)
    Wq = np.diag(s1) @ np.where(U >= 0, 1.0, -1.0) @ np.where(V >= 0, 1.0, -1.0).T @ np.diag(s2)
    np.testing.assert_allclose(S.forward(X, U, V, s1, s2), X @ Wq.T, rtol=1e-12, atol=1e-12)
    assert S.loss(X, Y, U, V, s1, s2) == pytest.approx(np.mean((X @ Wq.T - Y) ** 2), rel=1e-12)


def test_scale_gradients_match_finite_differences():
    X, Y, U, V, s1, s2 = _layer(2)
    _, _, ds1, ds2 = S.grads(X, Y, U, V, s1, s2)
    h = 1e-6
    for i in range(len(s1)):
        e = np.zeros_like(s1)
        e[i] = h
        fd = (S.loss(X, Y, U, V, s1 + e, s2) - S.loss(X, Y, U, V, s1 - e, s2)) / (2 * h)
        assert ds1[i] == pytest.approx(fd, rel=1e-6, abs=1e-10)
    for j in range(len(s2)):
        e = np.zeros_like(s2)
        e[j] = h
        fd = (S.loss(X, Y, U, V, s1, s2 + e) - S.loss(X, Y, U, V, s1, s2 - e)) / (2 * h)
        assert ds2[j] == pytest.approx(fd, rel=1e-6, abs=1e-10)


def test_latent_gradients_are_the_sign_gradients():
    # STE: dL/dU is the derivative of the loss in the sign matrix itself,
    # checked by finite differences with the signs made continuous
    X, Y, U, V, s1, s2 = _layer(3)
    dU, dV, _, _ = S.grads(X, Y, U, V, s1, s2)
    SU, SV = np.where(U >= 0, 1.0, -1.0), np.where(V >= 0, 1.0, -1.0)

    def f(SUc, SVc):
        Yq = (X * s2) @ SVc @ SUc.T * s1
        return np.mean((Yq - Y) ** 2)
    h = 1e-6
    for (i, k) in [(0, 0), (3, 2), (8, 3), (5, 1)]:
        E = np.zeros_like(SU)
        E[i, k] = h
        assert dU[i, k] == pytest.approx((f(SU + E, SV) - f(SU - E, SV)) / (2 * h), rel=1e-6, abs=1e-10)
    for (j, k) in [(0, 0), (10, 3), (4, 2)]:
        E = np.zeros_like(SV)
        E[j, k] = h
        assert dV[j, k] == pytest.approx((f(SU, SV + E) - f(SU, SV - E)) / (2 * h), rel=1e-6, abs=1e-10)
    # and they do not depend on the latents' magnitudes
    g2 = S.grads(X, Y, 3.0 * U, 0.5 * V, s1, s2)
    np.testing.assert_array_equal(g2[0], dU)
    np.testing.assert_array_equal(g2[1], dV)


def test_adam_matches_pytorch_and_a_hand_case():
    rng = np.random.default_rng(4)
    params = [rng.standard_normal((3, 2)), rng.standard_normal(5)]
    tp = [torch.tensor(p.copy(), dtype=torch.float64, requires_grad=True) for p in params]
    opt = torch.optim.Adam(tp, lr=1e-3)
    st = S.adam_init(params)
    for step in range(4):
        gs = [rng.standard_normal(p.shape) for p in params]
        for t, g in zip(tp, gs):
            t.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        params = S.adam_step(params, gs, st, 1e-3)
        for p, t in zip(params, tp):
            np.testing.assert_allclose(p, t.detach().numpy(), rtol=1e-13, atol=1e-15)
    # hand case: gradients 2 then -1 on a scalar at 0, lr 0.1:
    # step 1: m = 0.2, v = 0.004, mh = 2, vh = 4, p = -0.1 * 2 / (2 + 1e-8)
    # step 2: m = 0.18 - 0.1 = 0.08, v = 0.003996 + 0.001 = 0.004996,
    #         mh = 0.08 / 0.19, vh = 0.004996 / 0.001999
    p1 = -0.1 * 2.0 / (2.0 + 1e-8)
    p2 = p1 - 0.1 * (0.08 / 0.19) / (np.sqrt(0.004996 / 0.001999) + 1e-8)
    st = S.adam_init([np.zeros(1)])
    q = S.adam_step([np.zeros(1)], [np.array([2.0])], st, 0.1)
    assert q[0][0] == pytest.approx(p1, rel=1e-14)
    q = S.adam_step(q, [np.array([-1.0])], st, 0.1)
    assert q[0][0] == pytest.approx(p2, rel=1e-12)


def test_cosine_schedule_matches_pytorch():
    K = 37
    p = torch.zeros(1, requires_grad=True)
    opt = torch.optim.SGD([p], lr=1e-4)
    sch = torch.optim.lr_scheduler.CosineAnnealingLR(opt, T_max=K, eta_min=1e-6)
    for t in range(K):
        assert S.cosine_lr(t, K) == pytest.approx(opt.param_groups[0]["lr"], rel=1e-12)
        opt.step()
        sch.step()
    assert S.cosine_lr(0, K) == 1e-4
    assert S.cosine_lr(K, K) == pytest.approx(1e-6, rel=1e-12)


def test_planted_exact_layer_does_not_move():
    X, _, U, V, s1, s2 = _layer(5)
    Y = S.forward(X, U, V, s1, s2)            # the layer is exactly representable
    batches = [np.arange(0, 20), np.arange(20, 40), np.arange(0, 40)]
    U2, V2, a, b, losses = S.refine(X, Y, U, V, s1, s2, batches)
    assert max(losses) == 0.0
    np.testing.assert_array_equal(U2, U)
    np.testing.assert_array_equal(V2, V)
    np.testing.assert_array_equal(a, s1)
    np.testing.assert_array_equal(b, s2)


def test_refinement_descends_on_perturbed_scales():
    # signs right, scales off by up to 30 %: the loss falls steadily
    X, _, U, V, s1, s2 = _layer(6, T=200)
    Y = S.forward(X, U, V, s1, s2)
    rng = np.random.default_rng(7)
    a0 = s1 * rng.uniform(0.7, 1.3, s1.shape)
    b0 = s2 * rng.uniform(0.7, 1.3, s2.shape)
    batches = [np.arange(200)] * 60
    _, _, a, b, losses = S.refine(X, Y, U, V, a0, b0, batches, lr_max=1e-2, lr_min=3e-4)
    assert losses[-1] < 0.05 * losses[0]
    # Adam's steps are not monotone (the latents move too, and signs can
    # flip), but a small enough first step is a descent step
    _, _, _, _, l2 = S.refine(X, Y, U, V, a0, b0, [np.arange(200)] * 2, lr_max=1e-5, lr_min=1e-5)
    U1, V1, a1, b1, _ = S.refine(X, Y, U, V, a0, b0, [np.arange(200)], lr_max=1e-5, lr_min=1e-5)
    assert S.loss(X, Y, U1, V1, a1, b1) < l2[0]
