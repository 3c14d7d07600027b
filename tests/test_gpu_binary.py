"""GPU parity of the binary-layer product (nq_binary_matmul) and the sign
transpose (nq_transpose_signs) against the CPU oracle. One input runs the
lookup-table kernel, two or more the bf16 matrix-core kernel; the shapes
below cover both.

The transpose is bit-exact against oracle.lbadmm.pack_signs of the
transposed sign matrix. The product is compared with oracle.binary in
float64: the kernel sums +-x in float32 over n, then over r, so the bound
is a few float32 roundings of the sum of the absolute terms; the tests use a
relative Frobenius tolerance of 1e-5 (2e-5 at the full 8192 x 28672,
r = 6144 size).
"""
import numpy as np
import pytest

from oracle import binary as OB
from oracle import lbadmm as O
from synth import make_tiny

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


def bits_dev(S, dev):
    return T(O.pack_signs(S).view(np.int32), dev)


def layer(rng, m, n, r):
    SU = np.where(rng.random((m, r)) < 0.5, -1.0, 1.0)
    SV = np.where(rng.random((n, r)) < 0.5, -1.0, 1.0)
    s1 = rng.uniform(0.1, 2.0, m).astype(np.float32)
    s2 = rng.uniform(0.1, 2.0, n).astype(np.float32)
    return SU, SV, s1, s2


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 31), (64, 32), (65, 33), (200, 130), (1000, 97)])
def test_transpose_signs_bit_exact(gpu, rows, cols):
    import sub_bit_weight_lb_amd as nq
    rng = np.random.default_rng(rows * 7 + cols)
    S = np.where(rng.random((rows, cols)) < 0.5, -1.0, 1.0)
    print(f"case transpose {rows}x{cols}", flush=True)
    out = nq.transpose_signs(bits_dev(S, gpu), rows, cols)
    np.testing.assert_array_equal(H(out).view(np.uint32), O.pack_signs(S.T))
    back = nq.transpose_signs(out, cols, rows)
    np.testing.assert_array_equal(H(back).view(np.uint32), O.pack_signs(S))


@pytest.mark.parametrize("m,n,r,B", [(1, 1, 1, 1), (64, 48, 8, 1), (300, 200, 70, 3), (257, 1000, 33, 2),
                                     (100, 4100, 2049, 5), (4096, 4096, 2048, 1), (4096, 4096, 2048, 8),
                                     (11008, 4096, 1536, 4), (300, 200, 70, 9), (257, 1000, 33, 33),
                                     (65, 4100, 2049, 16), (4096, 4096, 2048, 24),
                                     (1, 1, 1, 2), (3, 5, 2, 17), (64, 33, 31, 100),
                                     (129, 129, 129, 31)])
def test_binary_matmul_matches_oracle(gpu, m, n, r, B):
    import sub_bit_weight_lb_amd as nq
    rng = np.random.default_rng(m + 3 * n + 7 * r + B)
    SU, SV, s1, s2 = layer(rng, m, n, r)
    X = rng.standard_normal((B, n)).astype(np.float32)
    print(f"case matmul m={m} n={n} r={r} B={B}", flush=True)
    Vt = nq.transpose_signs(bits_dev(SV, gpu), n, r)
    Y = H(nq.binary_matmul(bits_dev(SU, gpu), Vt, T(s1, gpu), T(s2, gpu), T(X, gpu), r))
    ref = OB.binary_matmul(X, O.pack_signs(SU), O.pack_signs(SV), r, s1, s2)
    assert Y.shape == ref.shape
    e = relerr(Y, ref)
    print(f"  rel err {e:.2e}", flush=True)
    assert e < 1e-5


def test_bf16_terms_are_exact(gpu):
    """Two or more inputs run on the bf16 matrix cores with each input split
    into three bf16 terms, which is exact: only the fp32 accumulation
    rounds. Over 4096 columns and 2048 ranks that keeps the product within
    about 5e-7 of the float64 oracle. Keeping only the first two terms
    would leave ~1e-5, only the first ~3e-3 (fp32 accumulation of the
    truncated terms, 32 columns per step, simulated in float64 on these
    sizes), so a 2e-6 bound tells them apart where the general 1e-5
    tolerance would not."""
    import sub_bit_weight_lb_amd as nq
    m, n, r, B = 1024, 4096, 2048, 16
    rng = np.random.default_rng(11)
    SU, SV, s1, s2 = layer(rng, m, n, r)
    X = rng.standard_normal((B, n)).astype(np.float32)
    print(f"case bf16 exactness m={m} n={n} r={r} B={B}", flush=True)
    Vt = nq.transpose_signs(bits_dev(SV, gpu), n, r)
    Y = H(nq.binary_matmul(bits_dev(SU, gpu), Vt, T(s1, gpu), T(s2, gpu), T(X, gpu), r))
    ref = OB.binary_matmul(X, O.pack_signs(SU), O.pack_signs(SV), r, s1, s2)
    assert relerr(Y, ref) < 2e-6


def test_binary_matmul_strided_vector_and_repeatable(gpu):
    """Row strides above the widths, a 1-D input, and bit-identical repeats
    (one input and three inputs take different kernel instances, so those
    two agree to rounding, not bit for bit)."""
    import torch
    import sub_bit_weight_lb_amd as nq
    rng = np.random.default_rng(5)
    m, n, r, B = 150, 300, 45, 3
    SU, SV, s1, s2 = layer(rng, m, n, r)
    X = rng.standard_normal((B, n)).astype(np.float32)
    ub = torch.zeros((m, 5), dtype=torch.int32, device=gpu)
    ub[:, :2] = bits_dev(SU, gpu)
    vt = torch.zeros((r, 12), dtype=torch.int32, device=gpu)
    nq.transpose_signs(bits_dev(SV, gpu), n, r, out=vt[:, :10])
    Xw = torch.zeros((B, n + 7), dtype=torch.float32, device=gpu)
    Xw[:, :n] = T(X, gpu)
    Yw = torch.full((B, m + 3), 7.0, dtype=torch.float32, device=gpu)
    nq.binary_matmul(ub[:, :2], vt[:, :10], T(s1, gpu), T(s2, gpu), Xw[:, :n], r, Y=Yw[:, :m])
    ref = OB.binary_matmul(X, O.pack_signs(SU), O.pack_signs(SV), r, s1, s2)
    assert relerr(H(Yw[:, :m]), ref) < 1e-5
    assert np.all(H(Yw[:, m:]) == 7.0)           # past the row width: untouched
    y1 = nq.binary_matmul(ub[:, :2], vt[:, :10], T(s1, gpu), T(s2, gpu), Xw[1, :n], r)
    assert y1.dim() == 1
    assert relerr(H(y1), ref[1]) < 1e-5
    y1b = nq.binary_matmul(ub[:, :2], vt[:, :10], T(s1, gpu), T(s2, gpu), Xw[1, :n], r)
    np.testing.assert_array_equal(H(y1), H(y1b))          # same call, same sums
    Yw2 = torch.empty((B, m), dtype=torch.float32, device=gpu)
    nq.binary_matmul(ub[:, :2], vt[:, :10], T(s1, gpu), T(s2, gpu), Xw[:, :n], r, Y=Yw2)
    np.testing.assert_array_equal(H(Yw2), H(Yw[:, :m]))


def test_binary_matmul_on_a_factorised_layer(gpu):
    """The run's own outputs (signs, scales) applied to inputs equal the
    product with the layer they describe, formed densely by the oracle."""
    import sub_bit_weight_lb_amd as nq
    L = make_tiny(192, 160, 40, seed=8, iters=4)
    m, n = L.W.shape
    res = nq.LBADMM(m, n, 40, iters=4, init_draws=True).run(T(L.W, gpu), T(L.d_out, gpu), T(L.d_in, gpu),
                                          T(L.EU, gpu), T(L.EV, gpu))
    Vt = nq.transpose_signs(res.V_bits, n, 40)
    X = np.random.default_rng(2).standard_normal((4, n)).astype(np.float32)
    Y = H(nq.binary_matmul(res.U_bits, Vt, res.s1, res.s2, T(X, gpu), 40))
    SU = O.unpack_signs(H(res.U_bits).view(np.uint32), 40)
    SV = O.unpack_signs(H(res.V_bits).view(np.uint32), 40)
    W_hat = O.reconstruct(H(res.s1).astype(np.float64), SU, SV, H(res.s2).astype(np.float64))
    assert relerr(Y, X.astype(np.float64) @ W_hat.T) < 1e-5


@pytest.mark.parametrize("B", [2, 16])
def test_binary_matmul_full_size_70b_down(gpu, B):
    """8192 x 28672 at r = 6144 (the largest layer), against the whole
    float64 oracle output: B = 2 (lookup-table kernel) and B = 16 (matrix
    cores)."""
    import sub_bit_weight_lb_amd as nq
    m, n, r = 8192, 28672, 6144
    rng = np.random.default_rng(70)
    SU, SV, s1, s2 = layer(rng, m, n, r)
    X = rng.standard_normal((B, n)).astype(np.float32)
    print(f"case matmul 8192x28672 r=6144 B={B}", flush=True)
    ub, vb = O.pack_signs(SU), O.pack_signs(SV)
    Vt = nq.transpose_signs(T(vb.view(np.int32), gpu), n, r)
    Y = H(nq.binary_matmul(T(ub.view(np.int32), gpu), Vt, T(s1, gpu), T(s2, gpu), T(X, gpu), r))
    ref = OB.binary_matmul(X, ub, vb, r, s1, s2)
    e = relerr(Y, ref)
    print(f"  rel err {e:.2e}", flush=True)
    assert e < 2e-5
