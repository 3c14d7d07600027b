"""GPU parity of the Ledoit-Wolf diagonal preconditioners (nq_lw_*) against
oracle/precond.py on the same seeded activation samples (synth.activations).

The GPU forms each chunk's Z^T Z on the fp32 matrix cores and accumulates
chunks in fp64; the oracle works in fp64 throughout. d is compared to 1e-5
relative and the shrinkage intensity to 1e-5 absolute (plus 1e-4 relative);
see check_d for how the shrinkage's rounding carries into d.
At 16384 x 4096 the oracle's per-sample sum is too slow, so d is checked
against the estimator's form d^2 = (1 - s) S_jj + s m with S_jj and m from
the inputs in fp64, and s against scikit-learn's ledoit_wolf (the library
form the oracle is pinned to on the CPU).
"""
import numpy as np
import pytest

from oracle import precond as P
from synth import make_activations

pytestmark = pytest.mark.gpu


def T(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def H(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("N, p, max_rows", [(300, 70, 16384), (1000, 256, 128), (4096, 130, 1000),
                                            (50, 200, 64), (1, 5, 1), (777, 33, 100)])
def test_lw_matches_oracle(gpu, N, p, max_rows):
    import sub_bit_weight_lb_amd as nq
    Z = make_activations(N, p, seed=N + p)
    print(f"case N={N} p={p} max_rows={max_rows}", flush=True)
    with nq.LedoitWolf(p, max_rows) as lw:
        lw.accumulate(T(Z, gpu))
        d, s = lw.finalize()
    check_d(H(d), s, Z)


def check_d(d, s, Z):
    """d and the shrinkage s against the oracle. The shrinkage to 1e-5
    absolute (+1e-4 relative): the GPU forms b2bar as sum ||z||^4 - N ||S||^2
    with S from fp32 products, which leaves ~1e-7 of rounding where the exact
    b2bar is 0 (one sample). d^2 = (1 - s) S_jj + s m moves by
    |s - s_ref| |m - S_jj| with the shrinkage, so d^2 is held to that plus
    2e-5 relative, and to its own s by the same formula to 2e-5."""
    d_ref, s_ref = P.diag_preconditioner(Z)
    assert abs(s - s_ref) <= 1e-5 + 1e-4 * s_ref, (s, s_ref)
    S = P.second_moment(Z)
    Sjj = np.diag(S)
    m = np.trace(S) / S.shape[0]
    d2 = d.astype(np.float64) ** 2
    np.testing.assert_allclose(d2, (1 - s) * Sjj + s * m, rtol=2e-5, atol=0)
    slack = abs(s - s_ref) * np.abs(m - Sjj) + 2e-5 * d_ref ** 2
    assert np.all(np.abs(d2 - d_ref ** 2) <= slack), np.max(np.abs(d2 - d_ref ** 2) - slack)


def test_lw_chunks_reset_and_strided_input(gpu):
    import torch
    import sub_bit_weight_lb_amd as nq
    N, p = 2000, 96
    Z = make_activations(N, p, seed=5)
    with nq.LedoitWolf(p, 512) as lw:
        # three calls of ragged sizes, one of them through a strided view
        wide = torch.zeros((700, p + 9), dtype=torch.float32, device=gpu)
        wide[:, :p] = T(Z[600:1300], gpu)
        lw.accumulate(T(Z[:600], gpu))
        lw.accumulate(wide[:, :p])
        lw.accumulate(T(Z[1300:], gpu))
        d1, s1 = lw.finalize()
        check_d(H(d1), s1, Z)
        # finalize keeps the statistics; reset forgets them
        d1b, s1b = lw.finalize()
        np.testing.assert_array_equal(H(d1b), H(d1))
        lw.reset()
        Z2 = make_activations(300, p, seed=6)
        lw.accumulate(T(Z2, gpu))
        d2, s2 = lw.finalize()
    check_d(H(d2), s2, Z2)
    # the same samples in one piece agree with the three pieces to rounding
    d3, _ = nq.ledoit_wolf_diag(T(Z, gpu))
    np.testing.assert_allclose(H(d3), H(d1), rtol=2e-6)


def test_lw_errors(gpu):
    import sub_bit_weight_lb_amd as nq
    with nq.LedoitWolf(8, 16) as lw:
        with pytest.raises(nq.NQError):
            lw.finalize()                      # nothing accumulated
        with pytest.raises(ValueError):
            lw.accumulate(T(np.zeros((4, 9), np.float32), gpu))
    with pytest.raises(nq.NQError):
        nq.LedoitWolf(0, 16)
    with pytest.raises(nq.NQError):
        nq.LedoitWolf(16385, 16)


def test_lw_feeds_the_factorisation(gpu):
    """d_out, d_in from an input and an output-side sample go straight into
    the run; its one-iteration state matches the oracle run with the same
    preconditioners."""
    import sub_bit_weight_lb_amd as nq
    from oracle import lbadmm as O
    m, n, r, N = 192, 256, 48, 1500
    rng = np.random.default_rng(12)
    W = (0.02 * rng.standard_normal((m, n))).astype(np.float32)
    X = make_activations(N, n, seed=13)
    Y = (X.astype(np.float64) @ W.T.astype(np.float64)).astype(np.float32)
    d_out, d_in = nq.preconditioners(T(X, gpu), T(Y, gpu))
    do_ref, di_ref = P.preconditioners(X, Y)
    np.testing.assert_allclose(H(d_out), do_ref, rtol=1e-5)
    np.testing.assert_allclose(H(d_in), di_ref, rtol=1e-5)
    EU = rng.standard_normal((m, r)).astype(np.float32)
    EV = rng.standard_normal((n, r)).astype(np.float32)
    h = nq.LBADMM(m, n, r, iters=1, balance=False, init_draws=True)
    h.run(T(W, gpu), d_out, d_in, T(EU, gpu), T(EV, gpu))
    st = {k: H(v) for k, v in h.state().items()}
    h.close()
    Wt = O.precondition(W, H(d_out), H(d_in))
    ref = O.iterate(Wt, O.init_state(Wt, r, 5, EU=EU, EV=EV), 1.0, 5, 1)
    for k in ("U", "V"):
        e = np.linalg.norm(st[k] - getattr(ref, k)) / np.linalg.norm(getattr(ref, k))
        assert e < 1e-4, (k, e)


def test_lw_full_size_chunked(gpu):
    """16384 tokens x 4096 features (the input width of a Llama-2-7B
    projection) in four chunks of 4096 rows."""
    from sklearn.covariance import ledoit_wolf
    import sub_bit_weight_lb_amd as nq
    N, p = 16384, 4096
    Z = make_activations(N, p, seed=99)
    print(f"case N={N} p={p}", flush=True)
    with nq.LedoitWolf(p, 4096) as lw:
        lw.accumulate(T(Z, gpu))
        d, s = lw.finalize()
    d = H(d).astype(np.float64)
    Z64 = Z.astype(np.float64)
    Sjj = np.einsum("kj,kj->j", Z64, Z64) / N
    m = Sjj.mean()
    np.testing.assert_allclose(d ** 2, (1 - s) * Sjj + s * m, rtol=2e-5)
    _, s_sk = ledoit_wolf(Z64, assume_centered=True)
    print(f"  shrinkage gpu {s:.8f} sklearn {s_sk:.8f}", flush=True)
    assert abs(s - s_sk) <= 1e-5 + 1e-4 * s_sk


def test_lw_wide_features(gpu):
    """11008 features (the output width of a Llama-2-7B MLP projection, past
    the ADMM path's largest rank), 640 tokens in chunks of 256 (the last
    ragged): the estimator's form with exact S_jj, and the intensity
    against scikit-learn."""
    from sklearn.covariance import ledoit_wolf
    import sub_bit_weight_lb_amd as nq
    N, p = 640, 11008
    Z = make_activations(N, p, seed=21)
    print(f"case N={N} p={p}", flush=True)
    with nq.LedoitWolf(p, 256) as lw:
        lw.accumulate(T(Z, gpu))
        d, s = lw.finalize()
    d = H(d).astype(np.float64)
    Z64 = Z.astype(np.float64)
    Sjj = np.einsum("kj,kj->j", Z64, Z64) / N
    m = Sjj.mean()
    np.testing.assert_allclose(d ** 2, (1 - s) * Sjj + s * m, rtol=2e-5)
    _, s_sk = ledoit_wolf(Z64, assume_centered=True)
    print(f"  shrinkage gpu {s:.8f} sklearn {s_sk:.8f}", flush=True)
    assert abs(s - s_sk) <= 1e-5 + 1e-4 * s_sk
