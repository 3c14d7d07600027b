"""GPU parity of each building block against the CPU oracle (or a library
routine computing the same quantity), through the C ABI."""
import numpy as np
import pytest

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


@pytest.mark.parametrize("m,n", [(1, 1), (7, 5), (256, 512), (300, 130), (1000, 333)])
def test_precondition_bit_exact(gpu, m, n):
    import sub_bit_weight_lb_amd as nq
    rng = np.random.default_rng(m * 7 + n)
    W = (rng.standard_normal((m, n)) * 0.02).astype(np.float32)
    do = rng.lognormal(0, .5, m).astype(np.float32)
    di = rng.lognormal(0, .5, n).astype(np.float32)
    got = H(nq.op_precondition(T(W, gpu), T(do, gpu), T(di, gpu)))
    np.testing.assert_array_equal(got, O.precondition(W, do, di, np.float32))


@pytest.mark.parametrize("rows,k,cols", [(128, 64, 128), (300, 70, 90), (1000, 517, 260),
                                         (512, 4096, 256), (8192, 2048, 384)])
def test_sign_gemm_is_exact(gpu, rows, k, cols):
    """C = A S^T with S = +-1 (the STE step's products through the sign
    matrices) against the float64 product. A is split into three exact bf16
    terms, so only the fp32 accumulation rounds: at K = 4096 the error is
    ~3e-7, where keeping two terms would leave ~1e-5 and one ~3e-3 (the
    same sums as the binary product's exactness test). C^T is the same
    numbers, transposed."""
    import sub_bit_weight_lb_amd as nq
    rng = np.random.default_rng(rows + 3 * k + 7 * cols)
    A = rng.standard_normal((rows, k)).astype(np.float32)
    S = np.where(rng.random((cols, k)) < 0.5, -1.0, 1.0).astype(np.float32)
    print(f"case sign gemm rows={rows} k={k} cols={cols}", flush=True)
    C, Ct = nq.op_sign_gemm(T(A, gpu), T(S, gpu), transposed=True)
    C, Ct = H(C), H(Ct)
    ref = A.astype(np.float64) @ S.astype(np.float64).T
    assert relerr(C, ref) < 2e-6
    np.testing.assert_array_equal(Ct, C.T)


# (4608, 512, 2048): 288 tiles of 256 x 128, one round of 256 and 32 tiles
# split 8 ways along K; (5000, 100, 1700): 280 tiles padded from a ragged
# shape, 24 split 4 ways (one K step each); (4096, 2048, 1536): 192 tiles,
# fewer than the 256 CUs, cut into 4 chunks of 16 K steps, 3 chunks per
# workgroup, so most tiles sum partials from two workgroups; (2000, 1111,
# 1000): 64 tiles from a ragged shape, 4 chunks each over 256 workgroups
@pytest.mark.parametrize("rows,k,cols", [(256, 32, 128), (300, 70, 90), (1000, 517, 260),
                                         (512, 4096, 256), (4608, 512, 2048), (5000, 100, 1700),
                                         (4096, 2048, 1536), (2000, 1111, 1000)])
def test_gemm_rhs(gpu, rows, k, cols):
    import sub_bit_weight_lb_amd as nq
    rng = np.random.default_rng(rows + k + cols)
    A = rng.standard_normal((rows, k)).astype(np.float32)
    B = rng.standard_normal((k, cols)).astype(np.float32)
    P = rng.standard_normal((rows, cols)).astype(np.float32)
    rho = 0.75
    got = H(nq.op_gemm_rhs(T(A, gpu), T(B, gpu), T(P, gpu), rho))
    ref = A.astype(np.float64) @ B.astype(np.float64) + rho * P.astype(np.float64)
    # fp32 accumulation bound: ~ sqrt(k) eps |A||B| per entry
    assert relerr(got, ref) < 2e-6 * np.sqrt(k / 32.0) + 1e-6


@pytest.mark.parametrize("rows,cols", [(64, 16), (300, 100), (4096, 256), (1024, 700)])
def test_gram(gpu, rows, cols):
    import sub_bit_weight_lb_amd as nq
    rng = np.random.default_rng(rows * 3 + cols)
    V = (rng.standard_normal((rows, cols)) * 0.05).astype(np.float32)
    got = H(nq.op_gram(T(V, gpu), 1.0))
    ref = O.gram(V.astype(np.float64), 1.0)
    assert relerr(got, ref) < 1e-5
    np.testing.assert_array_equal(got, got.T)   # exactly symmetric


@pytest.mark.parametrize("r", [1, 3, 64, 100, 128, 300, 640, 2048])
def test_cholesky_inverse(gpu, r):
    import sub_bit_weight_lb_amd as nq
    rng = np.random.default_rng(r)
    V = (rng.standard_normal((max(2 * r, 8), r)) * 0.1).astype(np.float32)
    G = O.gram(V.astype(np.float64), 1.0).astype(np.float32)
    L, Gi, info = nq.op_cholesky_inverse(T(G, gpu))
    assert info == 0
    L, Gi = H(L), H(Gi)
    G64 = G.astype(np.float64)
    assert np.all(np.triu(L, 1) == 0)
    assert relerr(L, O.cholesky(G64)) < 1e-5
    assert relerr(L.astype(np.float64) @ L.T.astype(np.float64), G64) < 1e-6
    assert relerr(Gi, np.linalg.inv(G64)) < 1e-5
    np.testing.assert_array_equal(Gi, Gi.T)


def test_cholesky_reports_indefinite(gpu):
    import sub_bit_weight_lb_amd as nq
    G = np.eye(130, dtype=np.float32)
    G[70, 70] = -1.0
    _, _, info = nq.op_cholesky_inverse(T(G, gpu))
    assert info == 71


@pytest.mark.parametrize("rows,cols,T_", [(4, 3, 1), (256, 128, 5), (300, 70, 5), (1000, 260, 3),
                                          (64, 17, 20)])
def test_svid(gpu, rows, cols, T_):
    import sub_bit_weight_lb_amd as nq
    rng = np.random.default_rng(rows + cols)
    X = rng.standard_normal((rows, cols)).astype(np.float32)
    X[rng.random(X.shape) < 0.01] = 0.0
    Z, a, b = nq.op_svid(T(X, gpu), T_)
    Zr, ar, br = O.svid(X.astype(np.float64), T_)
    assert relerr(H(a), ar) < 1e-5
    assert relerr(H(b), br) < 1e-5
    assert relerr(H(Z), Zr) < 1e-5
    # signs follow X exactly (x >= 0 -> +)
    assert np.all((H(Z) >= 0) == (X >= 0))


# shapes cover each launch layout: the slab held in registers (4096 x 2048,
# 4096 x 1536), streamed slabs (11264 x 1536, 4096 x 3072, 8192 x 6144),
# guarded column blocks (300 x 70, 1000 x 260) and a grid of 128 (256 x 128)
@pytest.mark.parametrize("rows,cols,T_", [(256, 128, 5), (300, 70, 5), (1000, 260, 3),
                                          (4096, 2048, 5), (4096, 1536, 5), (11264, 1536, 5),
                                          (4096, 3072, 5), (8192, 6144, 2)])
def test_svid_dual(gpu, rows, cols, T_):
    """X = U + Lam, Z = SVID_T(X), Lam' = X - Z against the oracle's SVID."""
    import sub_bit_weight_lb_amd as nq
    print(f"case svid_dual {rows}x{cols} T={T_}", flush=True)
    rng = np.random.default_rng(rows * 3 + cols)
    U = (0.05 * rng.standard_normal((rows, cols))).astype(np.float32)
    Lam = (0.01 * rng.standard_normal((rows, cols))).astype(np.float32)
    Z, Lo, a, b = nq.op_svid_dual(T(U, gpu), T(Lam, gpu), T_)
    X = U.astype(np.float64) + Lam.astype(np.float64)
    Zr, ar, br = O.svid(X, T_)
    assert relerr(H(a), ar) < 1e-5
    assert relerr(H(b), br) < 1e-5
    assert relerr(H(Z), Zr) < 1e-5
    assert relerr(H(Lo), X - Zr) < 1e-5
    # the sign of Z follows X = U + Lam as the GPU forms it (fp32 add)
    Xf = U + Lam
    assert np.all((H(Z) >= 0) == (Xf >= 0))


def test_svid_exact_sign_rank1(gpu):
    import sub_bit_weight_lb_amd as nq
    rng = np.random.default_rng(5)
    a = rng.uniform(0.1, 2, 200)
    b = rng.uniform(0.1, 2, 96)
    X = (np.where(rng.random((200, 96)) < .5, -1.0, 1.0) * np.outer(a, b)).astype(np.float32)
    Z, _, _ = nq.op_svid(T(X, gpu), 1)
    assert relerr(H(Z), X) < 1e-6


@pytest.mark.parametrize("rows,cols,ld", [(1, 1, 1), (5, 31, 31), (3, 64, 64), (7, 65, 70),
                                          (33, 2970, 2970), (256, 128, 130)])
def test_pack_signs_bit_exact(gpu, rows, cols, ld):
    import torch
    import sub_bit_weight_lb_amd as nq
    rng = np.random.default_rng(rows * 1000 + cols)
    Xf = rng.standard_normal((rows, ld)).astype(np.float32)
    Xf[rng.random(Xf.shape) < 0.05] = 0.0
    Xf[rng.random(Xf.shape) < 0.05] = -0.0
    X = T(Xf, gpu)[:, :cols]
    nw = (cols + 31) // 32
    bits = torch.full((rows, nw + 3), -1, dtype=torch.int32, device=gpu)
    nq.pack_signs(X, bits=bits)
    got = H(bits).view(np.uint32)
    np.testing.assert_array_equal(got[:, :nw], O.pack_signs(Xf[:, :cols]))
    assert np.all(got[:, nw:] == 0xFFFFFFFF)      # words beyond ceil(cols/32) untouched
