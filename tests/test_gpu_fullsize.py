"""GPU parity at the full sizes of the synthetic Llama-2-shaped layers, in the
launch configuration the benchmark times (overlapped streams, profiling
events and the error computation on).

- 4096 x 4096, r = 2048 and 11008 x 4096, r = 1536: one iteration against the
  float64 oracle element by element; the whole run against the oracle's
  end-of-run figures stored under tests/golden/ (written by
  tests/golden/make_lbadmm_final.py, which calls only oracle/).
- The seven layers of one Llama-2-7B-shaped block (q, k, v, o at 4096 x 4096,
  r = 2048; gate and up at 11008 x 4096 and down at 4096 x 11008, r = 2970,
  which pads to 3072 and so pins the chain to two XCDs): one iteration of q,
  gate and down against the oracle, and the 40-iteration run of every layer
  against its stored end-of-run figures.
- 8192 x 28672, r = 6144: the oracle cannot run an iteration in seconds here,
  so the initial SVID projections are compared in full, the first U-half
  solve through sampled entries of its normal equations U G = R (G and R
  built from the inputs by the oracle's routines), and the whole run against
  the stored end-of-run figures when they exist.
"""
import json
import os

import numpy as np
import pytest

from oracle import lbadmm as O
from synth import make_layer

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ATTN = "llama2-7b-attn-4096x4096-r2048"
BLOCK_ONE = ["llama2-7b-block.q_proj", "llama2-7b-block.gate_proj", "llama2-7b-block.down_proj"]
BLOCK_ALL = ["llama2-7b-block." + p for p in
             ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")]
MLP = "llama2-7b-mlp-11008x4096-r1536"
DOWN70 = "llama2-70b-down-8192x28672-r6144"


def T(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def H(t):
    return t.detach().cpu().numpy()


def relerr(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def masked_rel(g, o, X):
    """Relative Frobenius difference over entries with |X| > 1e-3 rms(X)."""
    rms = np.sqrt(np.mean(X.astype(np.float64) ** 2))
    mask = np.abs(X) > 1e-3 * rms
    return relerr(np.where(mask, g, 0), np.where(mask, o, 0))


def sign_agreement(g, o):
    rms = np.sqrt(np.mean(o ** 2))
    mask = np.abs(o) > 1e-3 * rms
    return float(np.mean((g[mask] >= 0) == (o[mask] >= 0)))


def bench_run(L, iters, dev):
    """One run with the handle settings the benchmark uses; returns the
    result and the (unbalanced) ADMM state."""
    import sub_bit_weight_lb_amd as nq
    wl = L.workload
    m, n = L.W.shape
    h = nq.LBADMM(m, n, wl.r, rho=wl.rho, iters=iters, svid_steps=wl.svid_steps,
                  compute_error=True, profile=True, init_draws=True)
    res = h.run(T(L.W, dev), T(L.d_out, dev), T(L.d_in, dev), T(L.EU, dev), T(L.EV, dev))
    st = {k: H(v) for k, v in h.state().items()}
    h.close()
    return res, st


def check_final_properties(res, r):
    """Bits are the signs of the returned latents; balancing held."""
    U, V = H(res.U), H(res.V)
    SU = O.unpack_signs(H(res.U_bits).view(np.uint32), r)
    SV = O.unpack_signs(H(res.V_bits).view(np.uint32), r)
    np.testing.assert_array_equal(SU, O.sgn(U))
    np.testing.assert_array_equal(SV, O.sgn(V))
    np.testing.assert_allclose(np.linalg.norm(U, axis=0), np.linalg.norm(V, axis=0), rtol=1e-4)
    s = res.stats
    assert s["potrf_info"] == 0 and s["nonfinite"] == 0


def check_fingerprints(res, g):
    """The stored end-of-run fingerprints of the balanced factors and scales.
    The fp32 run follows the fp64 oracle's trajectory only approximately
    (the errors agree to 1e-3 absolute), so norms and means are held to 0.5 %
    and the fractions of non-negative entries to 0.005 absolute: wide enough
    for that drift, far below what a lost balance, an unfolded
    preconditioner or a flipped sign convention would change."""
    U, V = H(res.U).astype(np.float64), H(res.V).astype(np.float64)
    got = {"U_fro": np.linalg.norm(U), "V_fro": np.linalg.norm(V),
           "s1_mean": float(np.mean(H(res.s1))), "s2_mean": float(np.mean(H(res.s2))),
           "U_pos_frac": float(np.mean(U >= 0)), "V_pos_frac": float(np.mean(V >= 0))}
    for k, v in got.items():
        print(f"  {k}: gpu {v:.6g} oracle {g[k]:.6g}", flush=True)
    for k in ("U_fro", "V_fro", "s1_mean", "s2_mean"):
        assert abs(got[k] - g[k]) <= 5e-3 * abs(g[k]), k
    for k in ("U_pos_frac", "V_pos_frac"):
        assert abs(got[k] - g[k]) <= 5e-3, k


def load_golden(name):
    path = os.path.join(GOLDEN, f"lbadmm_final_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        return json.load(f)


@pytest.mark.parametrize("name", [ATTN, MLP] + BLOCK_ONE)
def test_one_iteration_full_size(gpu, name):
    L = make_layer(name)
    wl = L.workload
    print(f"case {name}: one iteration", flush=True)
    _, st = bench_run(L, 1, gpu)
    Wt = O.precondition(L.W, L.d_out, L.d_in)
    ref = O.init_state(Wt, wl.r, wl.svid_steps, EU=L.EU, EV=L.EV)
    ref = O.iterate(Wt, ref, wl.rho, wl.svid_steps, 1)
    eu, ev = relerr(st["U"], ref.U), relerr(st["V"], ref.V)
    print(f"  U {eu:.2e} V {ev:.2e}", flush=True)
    assert eu < 1e-4 and ev < 1e-4
    XU = ref.Lam_U + ref.Z_U
    XV = ref.Lam_V + ref.Z_V
    for k, Xk in (("Z_U", XU), ("Lam_U", XU), ("Z_V", XV), ("Lam_V", XV)):
        e = masked_rel(st[k], getattr(ref, k), Xk)
        assert e < 1e-4, (k, e)
    assert sign_agreement(st["U"], ref.U) >= 0.999
    assert sign_agreement(st["V"], ref.V) >= 0.999


@pytest.mark.parametrize("method, steps", [("cg", 8), ("gd", 4)])
def test_iterative_solve_full_size_sampled(gpu, method, steps):
    """4096 x 4096, r = 2048 with the iterative solve: the first U-half's rows
    are independent systems u G = r, so sampled rows of the GPU's U after one
    iteration are compared with oracle.iterative_solve on those rows (G and R
    built from the inputs by the oracle's routines, warm start U0)."""
    import sub_bit_weight_lb_amd as nq
    L = make_layer(ATTN)
    wl = L.workload
    print(f"case {ATTN}: one iteration, {method} x{steps}", flush=True)
    h = nq.LBADMM(wl.m, wl.n, wl.r, rho=wl.rho, iters=1, svid_steps=wl.svid_steps,
                  solver=(method, steps), init_draws=True)
    h.run(T(L.W, gpu), T(L.d_out, gpu), T(L.d_in, gpu), T(L.EU, gpu), T(L.EV, gpu))
    U = H(h.state()["U"])
    h.close()
    Wt = O.precondition(L.W, L.d_out, L.d_in)
    s0 = O.init_scale(Wt, wl.r)
    U0 = s0 * L.EU.astype(np.float64)
    V0 = s0 * L.EV.astype(np.float64)
    ZU0, _, _ = O.svid(U0, wl.svid_steps)
    rows = np.random.default_rng(8).choice(wl.m, 16, replace=False)
    G = O.gram(V0, wl.rho)
    R = O.rhs(Wt[rows], V0, ZU0[rows], np.zeros((len(rows), wl.r)), wl.rho)
    ref = O.iterative_solve(R, G, U0[rows], steps, method)
    e = relerr(U[rows], ref)
    print(f"  sampled rows {e:.2e}", flush=True)
    assert e < 1e-4


@pytest.mark.parametrize("name", [ATTN, MLP] + BLOCK_ALL)
def test_full_run_vs_stored_oracle(gpu, name):
    g = load_golden(name)
    assert g is not None, f"missing tests/golden/lbadmm_final_{name}.json"
    L = make_layer(name)
    wl = L.workload
    assert (g["m"], g["n"], g["r"], g["iters"], g["seed"]) == (wl.m, wl.n, wl.r, wl.iters, wl.seed)
    print(f"case {name}: {wl.iters} iterations", flush=True)
    res, _ = bench_run(L, wl.iters, gpu)
    s = res.stats
    print(f"  gpu {s['rel_err_wtilde']:.6f} oracle {g['rel_err_wtilde']:.6f}", flush=True)
    assert abs(s["rel_err_wtilde"] - g["rel_err_wtilde"]) < 1e-3
    assert abs(s["rel_err_w"] - g["rel_err_w"]) < 1e-3
    assert abs(s["sigma0"] - g["sigma0"]) / g["sigma0"] < 1e-6
    check_final_properties(res, wl.r)
    check_fingerprints(res, g)


@pytest.fixture(scope="module")
def down70():
    return make_layer(DOWN70)


def test_70b_down_initial_projections(gpu, down70):
    L = down70
    wl = L.workload
    print(f"case {DOWN70}: init", flush=True)
    _, st = bench_run(L, 0, gpu)
    Wt = O.precondition(L.W, L.d_out, L.d_in)
    s0 = O.init_scale(Wt, wl.r)
    del Wt
    for k, E in (("U", L.EU), ("V", L.EV)):
        X = s0 * E.astype(np.float64)
        assert relerr(st[k], X) < 1e-6
        Z, _, _ = O.svid(X, wl.svid_steps)
        assert relerr(st[f"Z_{k}"], Z) < 1e-4, k
        del X, Z


def test_70b_down_first_solve_sampled(gpu, down70):
    """Sampled entries of U G = R for the first U-half, with G = V0^T V0 + rho I
    and R = Wt V0 + rho Z_U0 (Lam = 0 at the start) built from the inputs."""
    L = down70
    wl = L.workload
    print(f"case {DOWN70}: first solve", flush=True)
    _, st = bench_run(L, 1, gpu)
    U = st["U"]
    rng = np.random.default_rng(70)
    rows = rng.choice(wl.m, 12, replace=False)
    cols = rng.choice(wl.r, 12, replace=False)
    Wt = O.precondition(L.W, L.d_out, L.d_in)
    s0 = O.init_scale(Wt, wl.r)
    V0 = s0 * L.EV.astype(np.float64)
    ZU0, _, _ = O.svid(s0 * L.EU.astype(np.float64), wl.svid_steps)
    Gcols = V0.T @ V0[:, cols]                      # r x 12
    Gcols[cols, np.arange(len(cols))] += wl.rho
    R = Wt[rows] @ V0[:, cols] + wl.rho * ZU0[np.ix_(rows, cols)]
    lhs = U[rows].astype(np.float64) @ Gcols
    e = relerr(lhs, R)
    print(f"  normal-equation residual {e:.2e}", flush=True)
    assert e < 1e-4


def test_70b_down_full_run(gpu, down70):
    g = load_golden(DOWN70)
    L = down70
    wl = L.workload
    print(f"case {DOWN70}: {wl.iters} iterations", flush=True)
    res, _ = bench_run(L, wl.iters, gpu)
    check_final_properties(res, wl.r)
    if g is None:
        pytest.skip("stored oracle figures for the 8192 x 28672 layer not written yet "
                    "(tests/golden/make_lbadmm_final.py)")
    s = res.stats
    print(f"  gpu {s['rel_err_wtilde']:.6f} oracle {g['rel_err_wtilde']:.6f}", flush=True)
    assert abs(s["rel_err_wtilde"] - g["rel_err_wtilde"]) < 1e-3
    assert abs(s["rel_err_w"] - g["rel_err_w"]) < 1e-3
    assert abs(s["sigma0"] - g["sigma0"]) / g["sigma0"] < 1e-6
    check_fingerprints(res, g)
