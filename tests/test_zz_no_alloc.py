"""nq_binary_matmul_noalloc (the binary-layer product on the library's fixed
per-GPU scratch, for callers that cannot allocate) against nq_binary_matmul
(the same product on a caller-given workspace). Both run the same kernels in
the same order, so their outputs must agree bit for bit; both are also held
to the oracle's tolerance. Two calls in a row share the fixed scratch: the
second, smaller one must not see anything the first left there."""
import ctypes as C

import numpy as np
import pytest

from oracle import binary as OB
from oracle import lbadmm as O

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


def operands(seed, m, n, r, B, dev):
    rng = np.random.default_rng(seed)
    SU = np.where(rng.random((m, r)) < 0.5, -1.0, 1.0)
    SV = np.where(rng.random((n, r)) < 0.5, -1.0, 1.0)
    s1 = rng.uniform(0.1, 2.0, m).astype(np.float32)
    s2 = rng.uniform(0.1, 2.0, n).astype(np.float32)
    X = rng.standard_normal((B, n)).astype(np.float32)
    import sub_bit_weight_lb_amd as nq
    ub = T(O.pack_signs(SU).view(np.int32), dev)
    vt = nq.transpose_signs(T(O.pack_signs(SV).view(np.int32), dev), n, r)
    dev_ops = (ub, vt, T(s1, dev), T(s2, dev), T(X, dev))
    return dev_ops, (X, O.pack_signs(SU), O.pack_signs(SV), r, s1, s2)


def run_both(nq, ops, r, dev):
    import torch
    ub, vt, s1, s2, X = ops
    B, m = X.shape[0], ub.shape[0]
    Y_ref = nq.binary_matmul(ub, vt, s1, s2, X, r)
    Y = torch.full((B, m), float("nan"), dtype=torch.float32, device=dev)
    nq.binary_matmul_noalloc(ub, vt, s1, s2, X, r, Y)
    torch.cuda.synchronize()
    return H(Y), H(Y_ref)


# (m, n, r, B): two or more inputs take the matrix-core kernels, one the
# lookup-table kernels; each second case is smaller than its first
PAIRS = [
    ((1000, 2000, 512, 16), (300, 500, 100, 3)),
    ((700, 900, 200, 2), (130, 260, 40, 1)),
    ((2048, 4096, 2048, 64), (512, 1024, 256, 9)),
]


@pytest.mark.parametrize("first, second", PAIRS)
def test_noalloc_matches_workspace_entry_point_twice(gpu, first, second):
    import sub_bit_weight_lb_amd as nq
    for k, (m, n, r, B) in enumerate((first, second)):
        print(f"noalloc call {k}: m={m} n={n} r={r} B={B}", flush=True)
        ops, ref_args = operands(100 + k, m, n, r, B, gpu)
        Y, Y_ref = run_both(nq, ops, r, gpu)
        np.testing.assert_array_equal(Y, Y_ref)
        tol = 2e-5 if r * n > 4e6 else 1e-5
        assert relerr(Y, OB.binary_matmul(*ref_args)) < tol


def test_noalloc_at_its_limit_then_vector(gpu):
    """A workspace near the limit (2^23 floats: 512 more columns of rank
    would pass it), then a one-input call into a strided Y."""
    import torch
    import sub_bit_weight_lb_amd as nq
    m, n, r, B = 1024, 2048, 6656, 128
    assert nq.binary_matmul_work_floats(B, n, r) <= nq.NOALLOC_MAX_FLOATS
    assert nq.binary_matmul_work_floats(B, n, r + 512) > nq.NOALLOC_MAX_FLOATS
    print(f"noalloc at limit: m={m} n={n} r={r} B={B}", flush=True)
    ops, ref_args = operands(7, m, n, r, B, gpu)
    Y, Y_ref = run_both(nq, ops, r, gpu)
    np.testing.assert_array_equal(Y, Y_ref)
    rows = np.random.default_rng(1).choice(B, 4, replace=False)
    X, bu, bv, _, s1, s2 = ref_args
    assert relerr(Y[rows], OB.binary_matmul(X[rows], bu, bv, r, s1, s2)) < 2e-5
    ub, vt, s1d, s2d, Xd = ops
    Yw = torch.full((2, m + 5), 3.0, dtype=torch.float32, device=gpu)
    nq.binary_matmul_noalloc(ub, vt, s1d, s2d, Xd[5], r, Yw[1, :m])
    # one input runs the lookup-table kernels, not the matrix-core ones of
    # the 128-input call: compare with the workspace entry point on that input
    y_ref = H(nq.binary_matmul(ub, vt, s1d, s2d, Xd[5], r))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(H(Yw[1, :m]), y_ref)
    assert relerr(y_ref, OB.binary_matmul(X[5:6], bu, bv, r, s1, s2)[0]) < 2e-5
    assert np.all(H(Yw[0]) == 3.0) and np.all(H(Yw[1, m:]) == 3.0)


def test_noalloc_rejects_beyond_the_limit_without_touching_Y(gpu):
    import torch
    import sub_bit_weight_lb_amd as nq
    from sub_bit_weight_lb_amd import _lib
    m, n, r, B = 64, 64, 8192, 129
    assert nq.binary_matmul_work_floats(B, n, r) > nq.NOALLOC_MAX_FLOATS
    Y = torch.full((B, m), 5.0, dtype=torch.float32, device=gpu)
    with pytest.raises(ValueError, match="more than the fixed scratch"):
        nq.binary_matmul_noalloc(torch.zeros((m, 256), dtype=torch.int32, device=gpu),
                                 torch.zeros((r, 2), dtype=torch.int32, device=gpu),
                                 torch.ones(m, device=gpu), torch.ones(n, device=gpu),
                                 torch.zeros((B, n), device=gpu), r, Y)
    # the C entry point refuses it too, before any device work
    ub = torch.zeros((m, 256), dtype=torch.int32, device=gpu)
    vt = torch.zeros((r, 2), dtype=torch.int32, device=gpu)
    s = torch.ones(m, device=gpu)
    X = torch.zeros((B, n), device=gpu)
    p = lambda t: C.c_void_p(t.data_ptr())  # noqa: E731
    st = _lib.load().nq_binary_matmul_noalloc(p(ub), 256, p(vt), 2, m, n, r, p(s), p(s), p(X),
                                              B, n, p(Y), m, None)
    assert st == _lib.NQ_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert np.all(H(Y) == 5.0)
