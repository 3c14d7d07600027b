"""GPU parity of the whole per-layer path (nq_lbadmm_run) against the oracle."""
import numpy as np
import pytest

from oracle import lbadmm as O
from synth import make_layer, make_tiny

pytestmark = pytest.mark.gpu


def T(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def H(t):
    return t.detach().cpu().numpy()


def relerr(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def run_gpu(L, r, iters, dev, rho=1.0, T_=5, balance=True, init_exact=False, U0=None, V0=None):
    import sub_bit_weight_lb_amd as nq
    m, n = L.W.shape
    h = nq.LBADMM(m, n, r, rho=rho, iters=iters, svid_steps=T_, balance=balance,
                  init_draws=not init_exact)
    U0 = L.EU if U0 is None else U0
    V0 = L.EV if V0 is None else V0
    res = h.run(T(L.W, dev), T(L.d_out, dev), T(L.d_in, dev), T(U0, dev), T(V0, dev))
    state = {k: H(v) for k, v in h.state().items()}
    h.close()
    return res, state


def masked_rel(g, o, X):
    """Relative Frobenius difference over entries with |X| > 1e-3 rms(X)."""
    rms = np.sqrt(np.mean(X.astype(np.float64) ** 2))
    mask = np.abs(X) > 1e-3 * rms
    return relerr(np.where(mask, g, 0), np.where(mask, o, 0))


def sign_agreement(g, o):
    rms = np.sqrt(np.mean(o ** 2))
    mask = np.abs(o) > 1e-3 * rms
    return float(np.mean((g[mask] >= 0) == (o[mask] >= 0)))


@pytest.mark.parametrize("shape", [(256, 512, 128), (300, 200, 70), (64, 48, 8), (1, 1, 1)])
def test_init_and_one_iteration_state(gpu, shape):
    m, n, r = shape
    L = make_tiny(m, n, r, seed=11 + m)
    for iters in (0, 1):
        res, st = run_gpu(L, r, iters, gpu, balance=False)
        Wt = O.precondition(L.W, L.d_out, L.d_in)
        ref = O.init_state(Wt, r, 5, EU=L.EU, EV=L.EV)
        ref = O.iterate(Wt, ref, 1.0, 5, iters)
        print(f"case {shape} iters={iters}", flush=True)
        assert relerr(st["U"], ref.U) < 1e-4, relerr(st["U"], ref.U)
        assert relerr(st["V"], ref.V) < 1e-4, relerr(st["V"], ref.V)
        XU = ref.Lam_U + ref.Z_U
        XV = ref.Lam_V + ref.Z_V
        for k, Xk in (("Z_U", XU), ("Lam_U", XU), ("Z_V", XV), ("Lam_V", XV)):
            o = getattr(ref, k)
            if np.linalg.norm(o) == 0:
                assert np.max(np.abs(st[k])) < 1e-6
            else:
                assert masked_rel(st[k], o, Xk) < 1e-4, (k, masked_rel(st[k], o, Xk))
        assert sign_agreement(st["U"], ref.U) >= 0.999
        assert sign_agreement(st["V"], ref.V) >= 0.999


def test_tiny_workload_full_run(gpu):
    L = make_layer("tiny-256x512-r128")
    wl = L.workload
    res, st = run_gpu(L, wl.r, wl.iters, gpu, rho=wl.rho, T_=wl.svid_steps)
    ref = O.lbadmm(L.W, L.d_out, L.d_in, wl.r, wl.rho, wl.iters, wl.svid_steps, EU=L.EU, EV=L.EV)
    s = res.stats
    print(f"gpu err {s['rel_err_wtilde']:.6f} oracle {ref.rel_err_wt:.6f}", flush=True)
    assert abs(s["rel_err_wtilde"] - ref.rel_err_wt) < 1e-3
    assert abs(s["rel_err_w"] - ref.rel_err_w) < 1e-3
    assert s["potrf_info"] == 0 and s["nonfinite"] == 0
    assert abs(s["sigma0"] - ref.sigma0) / ref.sigma0 < 1e-6
    # the GPU's own error report equals the error of its own outputs, recomputed here
    SU = O.unpack_signs(H(res.U_bits).view(np.uint32), wl.r)
    SV = O.unpack_signs(H(res.V_bits).view(np.uint32), wl.r)
    e_w = O.rel_error(L.W, H(res.s1), SU, SV, H(res.s2))
    assert abs(e_w - s["rel_err_w"]) < 1e-5
    # the returned bits are the signs of the returned latents, and balancing held
    np.testing.assert_array_equal(SU, O.sgn(H(res.U)))
    np.testing.assert_array_equal(SV, O.sgn(H(res.V)))
    np.testing.assert_allclose(np.linalg.norm(H(res.U), axis=0), np.linalg.norm(H(res.V), axis=0),
                               rtol=1e-4)
    assert sign_agreement(H(res.U), ref.U) > 0.95


def test_planted_fixed_point(gpu):
    m, n, r = 256, 384, 32
    rng = np.random.default_rng(3)
    s1 = rng.uniform(0.5, 2, m)
    s2 = rng.uniform(0.5, 2, n)
    SU = np.where(rng.random((m, r)) < .5, -1.0, 1.0)
    SV = np.where(rng.random((n, r)) < .5, -1.0, 1.0)
    W = O.reconstruct(s1, SU, SV, s2).astype(np.float32)
    import types
    L = types.SimpleNamespace(W=W, d_out=np.ones(m, np.float32), d_in=np.ones(n, np.float32))
    U0 = (s1[:, None] * SU).astype(np.float32)
    V0 = (s2[:, None] * SV).astype(np.float32)
    res, st = run_gpu(L, r, 10, gpu, init_exact=True, U0=U0, V0=V0)
    assert res.stats["rel_err_wtilde"] < 1e-5
    np.testing.assert_array_equal(O.unpack_signs(H(res.U_bits).view(np.uint32), r), SU)
    np.testing.assert_array_equal(O.unpack_signs(H(res.V_bits).view(np.uint32), r), SV)


def test_deterministic_rerun(gpu):
    import sub_bit_weight_lb_amd as nq
    L = make_tiny(300, 260, 70, seed=4, iters=3)
    h = nq.LBADMM(300, 260, 70, iters=3, init_draws=True)
    a = h.run(T(L.W, gpu), T(L.d_out, gpu), T(L.d_in, gpu), T(L.EU, gpu), T(L.EV, gpu))
    b = h.run(T(L.W, gpu), T(L.d_out, gpu), T(L.d_in, gpu), T(L.EU, gpu), T(L.EV, gpu))
    h.close()
    for x, y in ((a.U, b.U), (a.V, b.V), (a.s1, b.s1), (a.U_bits, b.U_bits)):
        np.testing.assert_array_equal(H(x), H(y))
    assert a.stats["rel_err_wtilde"] == b.stats["rel_err_wtilde"]


def test_bad_inputs_reported(gpu):
    import sub_bit_weight_lb_amd as nq
    L = make_tiny(64, 64, 8, seed=2)
    W = L.W.copy()
    W[3, 5] = np.nan
    with pytest.raises(nq.NQError, match="NONFINITE"):
        run_gpu(type("L", (), dict(W=W, d_out=L.d_out, d_in=L.d_in, EU=L.EU, EV=L.EV)), 8, 1, gpu)
    d = L.d_in.copy()
    d[7] = 0.0
    with pytest.raises(nq.NQError, match="BAD_PRECONDITIONER"):
        run_gpu(type("L", (), dict(W=L.W, d_out=L.d_out, d_in=d, EU=L.EU, EV=L.EV)), 8, 1, gpu)


@pytest.mark.parametrize("profile", [True, "rhs"])
def test_profile_phases(gpu, profile):
    """Every phase is timed with profile=True; with profile="rhs" only the
    RHS GEMM (one interval per half-iteration). Results do not depend on it."""
    import sub_bit_weight_lb_amd as nq
    L = make_tiny(300, 260, 70, seed=4, iters=3)
    h = nq.LBADMM(300, 260, 70, iters=3, profile=profile, init_draws=True)
    res = h.run(T(L.W, gpu), T(L.d_out, gpu), T(L.d_in, gpu), T(L.EU, gpu), T(L.EV, gpu))
    prof = h.profile(reset=True)
    h.close()
    assert prof["gemm_rhs"][1] == 2 * 3 and prof["gemm_rhs"][0] > 0.0
    others = ("gemm_solve", "chain", "svid", "prep", "finish")
    if profile == "rhs":
        assert all(prof[p][1] == 0 for p in others)
    else:
        assert all(prof[p][1] > 0 for p in others)
    plain, _ = run_gpu(L, 70, 3, gpu)
    np.testing.assert_array_equal(H(res.U), H(plain.U))


@pytest.mark.parametrize("shape", [(512, 384, 1100), (768, 640, 300), (512, 384, 2100)])
def test_launch_layouts_agree(gpu, shape, monkeypatch):
    """The pinned overlap (the chain's diagonal work on the last one or two
    XCDs, the RHS GEMM on the others with leftover tiles split along K), the
    unpinned overlap and the single-stream order compute the same iteration.
    r = 2100 pads to 2176 (34 diagonal workgroups per launch), which takes two
    XCDs by default; NQ_PIN=2 asks for two where one would do."""
    import sub_bit_weight_lb_amd as nq
    m, n, r = shape
    L = make_tiny(m, n, r, seed=21 + r, iters=2)
    outs = {}
    for name, env, single in (("default", None, False), ("two-xcds", "2", False),
                              ("unpinned", "0", False), ("single", None, True)):
        if env is None:
            monkeypatch.delenv("NQ_PIN", raising=False)
        else:
            monkeypatch.setenv("NQ_PIN", env)
        h = nq.LBADMM(m, n, r, iters=2, single_stream=single, init_draws=True)
        res = h.run(T(L.W, gpu), T(L.d_out, gpu), T(L.d_in, gpu), T(L.EU, gpu), T(L.EV, gpu))
        outs[name] = {k: H(v) for k, v in h.state().items()}
        h.close()
        print(f"case {shape} layout {name}: err {res.stats['rel_err_wtilde']:.6f}", flush=True)
    Wt = O.precondition(L.W, L.d_out, L.d_in)
    ref = O.iterate(Wt, O.init_state(Wt, r, 5, EU=L.EU, EV=L.EV), 1.0, 5, 2)
    for name, st in outs.items():
        assert relerr(st["U"], ref.U) < 1e-4, (name, relerr(st["U"], ref.U))
        assert relerr(st["V"], ref.V) < 1e-4, (name, relerr(st["V"], ref.V))
        for k in ("U", "V", "Lam_U", "Lam_V"):
            assert relerr(st[k], outs["single"][k]) < 2e-5, (name, k, relerr(st[k], outs["single"][k]))


@pytest.mark.parametrize("shape, seed", [((64, 48, 8), 7), ((300, 200, 70), 0x1234567890ab),
                                         ((1, 1, 1), 3)])
def test_builtin_philox_start(gpu, shape, seed):
    """U0 = V0 = NULL: the start is sigma0 times the library's Philox4x32-10
    normals, compared with the tests' own generator (tests/philox_cpu.py,
    pinned to the published known-answer vectors) to within one float32 ulp;
    sigma0 against the oracle."""
    import sub_bit_weight_lb_amd as nq
    from philox_cpu import normals
    m, n, r = shape
    L = make_tiny(m, n, r, seed=21 + m)
    print(f"case philox {shape} seed={seed:#x}", flush=True)
    h = nq.LBADMM(m, n, r, iters=0, seed=seed, balance=False)
    res = h.run(T(L.W, gpu), T(L.d_out, gpu), T(L.d_in, gpu))
    st = {k: H(v) for k, v in h.state().items()}
    h.close()
    s0 = res.stats["sigma0"]
    Wt = O.precondition(L.W, L.d_out, L.d_in)
    assert abs(s0 - O.init_scale(Wt, r)) / O.init_scale(Wt, r) < 1e-6
    for k, rows, stream in (("U", m, 0), ("V", n, 1)):
        z = normals(seed, stream, rows * r).reshape(rows, r)
        want = np.float32(s0) * z.astype(np.float32)
        got = st[k]
        ulp = np.spacing(np.abs(want).astype(np.float32))
        bad = np.abs(got - want) > ulp
        assert not bad.any(), (k, int(bad.sum()), got[bad][:4], want[bad][:4])


def test_finish_matches_oracle_on_gpu_state(gpu):
    """The balanced factors, scales and bits the run returns against
    oracle.finish applied to the GPU's own pre-balance state (get_state), so
    that the finish is checked element by element apart from the iterations."""
    import sub_bit_weight_lb_amd as nq
    L = make_tiny(300, 260, 70, seed=9, iters=3)
    m, n = L.W.shape
    r = 70
    h = nq.LBADMM(m, n, r, iters=3, init_draws=True)
    res = h.run(T(L.W, gpu), T(L.d_out, gpu), T(L.d_in, gpu), T(L.EU, gpu), T(L.EV, gpu))
    st = {k: H(v).astype(np.float64) for k, v in h.state().items()}
    h.close()
    Wt = O.precondition(L.W, L.d_out, L.d_in)
    Ub, Vb, s1, s2, _, _, ub, vb, e_wt, e_w = O.finish(
        Wt, L.W.astype(np.float64), L.d_out, L.d_in, st["U"], st["V"])
    for name, g, o in (("U", H(res.U), Ub), ("V", H(res.V), Vb)):
        rms = np.sqrt(np.mean(o ** 2))
        np.testing.assert_allclose(g, o, rtol=1e-5, atol=1e-6 * rms, err_msg=name)
    np.testing.assert_allclose(H(res.s1), s1, rtol=1e-5, atol=0)
    np.testing.assert_allclose(H(res.s2), s2, rtol=1e-5, atol=0)
    np.testing.assert_array_equal(H(res.U_bits).view(np.uint32), ub)
    np.testing.assert_array_equal(H(res.V_bits).view(np.uint32), vb)
    assert abs(res.stats["rel_err_wtilde"] - e_wt) < 1e-5
    assert abs(res.stats["rel_err_w"] - e_w) < 1e-5


@pytest.mark.parametrize("method, steps, shape", [("cg", 5, (256, 512, 128)),
                                                  ("gd", 3, (300, 200, 70)),
                                                  ("cg", 1, (64, 48, 8)),
                                                  ("cg", 12, (256, 384, 96)),
                                                  ("gd", 8, (1, 1, 1))])
def test_iterative_solve_iterations(gpu, method, steps, shape):
    """NQ_FLAG_SOLVE_CG / _GD: one and two iterations with the iterative solve
    against oracle.iterate with the same solver, warm start and step count."""
    import sub_bit_weight_lb_amd as nq
    m, n, r = shape
    L = make_tiny(m, n, r, seed=31 + m)
    Wt = O.precondition(L.W, L.d_out, L.d_in)
    for iters in (1, 2):
        print(f"case {method} x{steps} {shape} iters={iters}", flush=True)
        h = nq.LBADMM(m, n, r, iters=iters, balance=False, solver=(method, steps),
                      init_draws=True)
        h.run(T(L.W, gpu), T(L.d_out, gpu), T(L.d_in, gpu), T(L.EU, gpu), T(L.EV, gpu))
        st = {k: H(v) for k, v in h.state().items()}
        h.close()
        ref = O.init_state(Wt, r, 5, EU=L.EU, EV=L.EV)
        ref = O.iterate(Wt, ref, 1.0, 5, iters, solver=(method, steps))
        assert relerr(st["U"], ref.U) < 1e-4, relerr(st["U"], ref.U)
        assert relerr(st["V"], ref.V) < 1e-4, relerr(st["V"], ref.V)
        for k, Xk in (("Z_U", ref.Lam_U + ref.Z_U), ("Lam_U", ref.Lam_U + ref.Z_U),
                      ("Z_V", ref.Lam_V + ref.Z_V), ("Lam_V", ref.Lam_V + ref.Z_V)):
            assert masked_rel(st[k], getattr(ref, k), Xk) < 1e-4, k
        assert sign_agreement(st["U"], ref.U) >= 0.999


def test_iterative_solve_rejects_bad_desc(gpu):
    import sub_bit_weight_lb_amd as nq
    with pytest.raises(ValueError):
        nq.LBADMM(64, 48, 8, solver=("sor", 3))
    with pytest.raises(nq.NQError):
        nq.LBADMM(64, 48, 8, solver=("cg", 0))
    with pytest.raises(nq.NQError):
        nq.lbadmm_create(64, 48, 8, flags=nq.NQ_FLAG_SOLVE_CG | nq.NQ_FLAG_SOLVE_GD,
                         solve_steps=3)
    with pytest.raises(nq.NQError):
        nq.lbadmm_create(64, 48, 8, solve_steps=3)


def test_warm_start_is_taken_as_given(gpu):
    """Without NQ_FLAG_INIT_DRAWS, U0 and V0 are the starting latents: at
    iters = 0 the state holds them bit for bit and Z = SVID(U0), SVID(V0);
    with the flag the same arrays are draws scaled by sigma0."""
    import sub_bit_weight_lb_amd as nq
    m, n, r = 200, 150, 40
    L = make_tiny(m, n, r, seed=17)
    rng = np.random.default_rng(5)
    U0 = (0.05 * rng.standard_normal((m, r))).astype(np.float32)
    V0 = (0.05 * rng.standard_normal((n, r))).astype(np.float32)
    args = (T(L.W, gpu), T(L.d_out, gpu), T(L.d_in, gpu), T(U0, gpu), T(V0, gpu))
    Wt = O.precondition(L.W, L.d_out, L.d_in)
    for draws in (False, True):
        h = nq.LBADMM(m, n, r, iters=0, balance=False, init_draws=draws)
        res = h.run(*args)
        st = {k: H(v) for k, v in h.state().items()}
        h.close()
        if draws:
            s0 = np.float32(res.stats["sigma0"])
            np.testing.assert_array_equal(st["U"], s0 * U0)
            np.testing.assert_array_equal(st["V"], s0 * V0)
            ref = O.init_state(Wt, r, 5, EU=U0, EV=V0)
        else:
            np.testing.assert_array_equal(st["U"], U0)
            np.testing.assert_array_equal(st["V"], V0)
            ref = O.init_state(Wt, r, 5, U0=U0, V0=V0)
        for k, X in (("Z_U", ref.U), ("Z_V", ref.V)):
            assert masked_rel(st[k], getattr(ref, k), X) < 1e-4, (draws, k)
