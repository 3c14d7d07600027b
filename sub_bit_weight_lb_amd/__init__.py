"""LB-ADMM low-rank binary factorisation on MI355X (gfx950).

Thin Python binding of the C ABI in include/nq.h. Every step of the
per-layer path runs in the HIP kernels of libnq.so; this module only checks
and marshals arguments (torch tensors supply device memory and the current
stream). Importing works without a GPU; calls that need the device fail
loudly when libnq.so or the GPU is missing. There is no CPU fallback.

Functions mirror the C names without the ``nq_`` prefix:
    lbadmm_create / lbadmm_run / lbadmm_query / lbadmm_get_state /
    lbadmm_destroy / lbadmm_workspace_bytes / pack_signs /
    transpose_signs / binary_matmul /
    op_precondition / op_gram / op_gemm_rhs / op_cholesky_inverse / op_svid
plus the conveniences ``LBADMM`` (a handle object) and ``lbadmm`` (one call).
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional

from . import _lib
from ._lib import (NQ_FLAG_COMPUTE_ERROR, NQ_FLAG_INIT_EXACT, NQ_FLAG_NO_BALANCE,  # noqa: F401
                   NQ_FLAG_PROFILE, NQ_FLAG_PROFILE_RHS_ONLY, NQ_FLAG_SINGLE_STREAM, NQ_OK,
                   PHASES, Desc, Stats)

__all__ = [
    "NQError", "lbadmm_create", "lbadmm_run", "lbadmm_query", "lbadmm_get_state",
    "lbadmm_destroy", "lbadmm_profile", "lbadmm_workspace_bytes", "pack_signs", "transpose_signs",
    "binary_matmul", "op_precondition", "op_gram",
    "op_gemm_rhs", "op_cholesky_inverse", "op_svid", "LBADMM", "lbadmm", "Result",
    "status_string", "version",
]


class NQError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib.load()
        name = lib.nq_status_string(status).decode()
        msg = lib.nq_last_error_message().decode()
        super().__init__(f"{where}: {name}: {msg}")
        self.status = status


def _check(status: int, where: str):
    if status != NQ_OK:
        raise NQError(status, where)


def _torch():
    import torch
    return torch


def _ptr(t, name, dtype=None, ndim=None, allow_none=False, need_contig=True):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    if need_contig and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return C.c_void_p(int(stream))
    return C.c_void_p(_torch().cuda.current_stream().cuda_stream)


def status_string(status: int) -> str:
    return _lib.load().nq_status_string(status).decode()


def version() -> int:
    return int(_lib.load().nq_version())


def _desc(m, n, r, rho, iters, svid_steps, seed, flags) -> Desc:
    return Desc(int(m), int(n), int(r), float(rho), int(iters), int(svid_steps), int(seed),
                int(flags))


def lbadmm_workspace_bytes(m, n, r, rho=1.0, iters=50, svid_steps=5, seed=0, flags=0) -> int:
    out = C.c_size_t(0)
    d = _desc(m, n, r, rho, iters, svid_steps, seed, flags)
    _check(_lib.load().nq_lbadmm_workspace_bytes(C.byref(d), C.byref(out)),
           "nq_lbadmm_workspace_bytes")
    return int(out.value)


def lbadmm_create(m, n, r, rho=1.0, iters=50, svid_steps=5, seed=0,
                  flags=NQ_FLAG_COMPUTE_ERROR) -> int:
    h = C.c_void_p(0)
    d = _desc(m, n, r, rho, iters, svid_steps, seed, flags)
    _check(_lib.load().nq_lbadmm_create(C.byref(d), C.byref(h)), "nq_lbadmm_create")
    return h.value


def _stats_dict(s: Stats) -> dict:
    return {f: getattr(s, f) for f, _ in Stats._fields_ if f != "reserved"}


def lbadmm_run(h, W, d_out, d_in, U0=None, V0=None, U=None, V=None, s1=None, s2=None,
               U_bits=None, V_bits=None, want_stats=True, stream=None):
    """Enqueue one full per-layer run. Returns the stats dict when want_stats
    (the call then waits for the stream), else None."""
    torch = _torch()
    f32 = torch.float32
    if W is None or W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be a 2-D tensor with unit column stride")
    pW = _ptr(W, "W", f32, 2, need_contig=False)
    st = Stats()
    status = _lib.load().nq_lbadmm_run(
        C.c_void_p(h), pW, W.stride(0), _ptr(d_out, "d_out", f32, 1), _ptr(d_in, "d_in", f32, 1),
        _ptr(U0, "U0", f32, 2, True), _ptr(V0, "V0", f32, 2, True),
        _ptr(U, "U", f32, 2, True), _ptr(V, "V", f32, 2, True),
        _ptr(s1, "s1", f32, 1, True), _ptr(s2, "s2", f32, 1, True),
        _ptr(U_bits, "U_bits", torch.int32, 2, True), _ptr(V_bits, "V_bits", torch.int32, 2, True),
        C.byref(st) if want_stats else None, _stream(stream))
    _check(status, "nq_lbadmm_run")
    return _stats_dict(st) if want_stats else None


def lbadmm_query(h):
    st = Stats()
    status = _lib.load().nq_lbadmm_query(C.c_void_p(h), C.byref(st))
    return status, _stats_dict(st)


def lbadmm_get_state(h, U=None, V=None, Z_U=None, Lam_U=None, Z_V=None, Lam_V=None, stream=None):
    f32 = _torch().float32
    _check(_lib.load().nq_lbadmm_get_state(
        C.c_void_p(h), _ptr(U, "U", f32, 2, True), _ptr(V, "V", f32, 2, True),
        _ptr(Z_U, "Z_U", f32, 2, True), _ptr(Lam_U, "Lam_U", f32, 2, True),
        _ptr(Z_V, "Z_V", f32, 2, True), _ptr(Lam_V, "Lam_V", f32, 2, True), _stream(stream)),
        "nq_lbadmm_get_state")


def lbadmm_profile(h, reset=False) -> dict:
    """Per-phase device time under NQ_FLAG_PROFILE: {phase: (total_ms, intervals)}."""
    n = len(PHASES)
    ms = (C.c_double * n)()
    cnt = (C.c_int64 * n)()
    _check(_lib.load().nq_lbadmm_profile(C.c_void_p(h), ms, cnt, 1 if reset else 0),
           "nq_lbadmm_profile")
    return {p: (float(ms[i]), int(cnt[i])) for i, p in enumerate(PHASES)}


def lbadmm_destroy(h):
    if h:
        _lib.load().nq_lbadmm_destroy(C.c_void_p(h))


def pack_signs(X, bits=None, stream=None):
    """Sign bits of a 2-D float32 tensor (unit column stride): int32 words,
    bit k of word w of row i = [X[i, 32 w + k] >= 0]."""
    torch = _torch()
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    rows, cols = X.shape
    nw = (cols + 31) // 32
    if bits is None:
        bits = torch.empty((rows, nw), dtype=torch.int32, device=X.device)
    _check(_lib.load().nq_pack_signs(
        _ptr(X, "X", torch.float32, 2, need_contig=False), rows, cols, X.stride(0),
        _ptr(bits, "bits", torch.int32, 2, need_contig=False), bits.stride(0), _stream(stream)),
        "nq_pack_signs")
    return bits


def transpose_signs(bits, rows, cols, out=None, stream=None):
    """Sign bits of the transpose: bits holds rows x cols signs (int32 words,
    rows x ceil(cols/32) or wider, unit column stride); returns (or fills) the
    cols x ceil(rows/32) words of the cols x rows transpose."""
    torch = _torch()
    if bits.dim() != 2 or bits.stride(1) != 1 or bits.shape[0] != rows:
        raise ValueError("bits must be 2-D, rows x words, unit column stride")
    if out is None:
        out = torch.empty((cols, (rows + 31) // 32), dtype=torch.int32, device=bits.device)
    _check(_lib.load().nq_transpose_signs(
        _ptr(bits, "bits", torch.int32, 2, need_contig=False), rows, cols, bits.stride(0),
        _ptr(out, "out", torch.int32, 2, need_contig=False), out.stride(0), _stream(stream)),
        "nq_transpose_signs")
    return out


def binary_matmul(U_bits, Vt_bits, s1, s2, X, r, Y=None, work=None, stream=None):
    """Y = X W^T for the factorised layer W = diag(s1) S_U S_V^T diag(s2):
    U_bits (m x ceil(r/32) int32), Vt_bits (r x ceil(n/32) int32, from
    transpose_signs of the run's V_bits), s1 (m), s2 (n), X (B x n float32,
    or a vector of length n); work, if given, holds 8 B r float32. Returns Y
    (B x m, or length m)."""
    torch = _torch()
    vec = X.dim() == 1
    X2 = X.unsqueeze(0) if vec else X
    if X2.dim() != 2 or X2.stride(1) != 1:
        raise ValueError("X must be 1-D or 2-D with unit column stride")
    B, n = X2.shape
    m = U_bits.shape[0]
    if Vt_bits.shape[0] != r or s1.numel() != m or s2.numel() != n:
        raise ValueError("shapes of U_bits, Vt_bits, s1, s2 and X do not agree")
    if Y is None:
        Y = torch.empty((B, m), dtype=torch.float32, device=X.device)
    if work is None:
        work = torch.empty((max(8 * B * r, 1),), dtype=torch.float32, device=X.device)
    _check(_lib.load().nq_binary_matmul(
        _ptr(U_bits, "U_bits", torch.int32, 2, need_contig=False), U_bits.stride(0),
        _ptr(Vt_bits, "Vt_bits", torch.int32, 2, need_contig=False), Vt_bits.stride(0),
        m, n, r, _ptr(s1, "s1", torch.float32), _ptr(s2, "s2", torch.float32),
        _ptr(X2, "X", torch.float32, 2, need_contig=False), B, X2.stride(0),
        _ptr(Y, "Y", torch.float32, 2, need_contig=False), Y.stride(0),
        _ptr(work, "work", torch.float32), _stream(stream)), "nq_binary_matmul")
    return Y[0] if vec else Y


def op_precondition(W, d_out, d_in, stream=None):
    torch = _torch()
    m, n = W.shape
    out = torch.empty((m, n), dtype=torch.float32, device=W.device)
    f32 = torch.float32
    _check(_lib.load().nq_op_precondition(
        _ptr(W, "W", f32, 2), n, m, n, _ptr(d_out, "d_out", f32, 1), _ptr(d_in, "d_in", f32, 1),
        _ptr(out, "Wt", f32, 2), n, _stream(stream)), "nq_op_precondition")
    return out


def op_gram(A, rho, stream=None):
    torch = _torch()
    rows, cols = A.shape
    G = torch.empty((cols, cols), dtype=torch.float32, device=A.device)
    _check(_lib.load().nq_op_gram(_ptr(A, "A", torch.float32, 2), rows, cols, cols, float(rho),
                                  _ptr(G, "G", torch.float32, 2), cols, _stream(stream)),
           "nq_op_gram")
    return G


def op_gemm_rhs(A, B, P=None, rho=0.0, stream=None):
    torch = _torch()
    rows, k = A.shape
    k2, cols = B.shape
    if k2 != k:
        raise ValueError("inner dimensions differ")
    Cm = torch.empty((rows, cols), dtype=torch.float32, device=A.device)
    f32 = torch.float32
    _check(_lib.load().nq_op_gemm_rhs(
        _ptr(A, "A", f32, 2), k, _ptr(B, "B", f32, 2), cols, _ptr(P, "P", f32, 2, True), cols,
        float(rho), _ptr(Cm, "C", f32, 2), cols, rows, cols, k, _stream(stream)), "nq_op_gemm_rhs")
    return Cm


def op_cholesky_inverse(G, stream=None):
    """Returns (L, Ginv, info); raises NQError on a non-positive pivot."""
    torch = _torch()
    r = G.shape[0]
    L = torch.empty((r, r), dtype=torch.float32, device=G.device)
    Gi = torch.empty((r, r), dtype=torch.float32, device=G.device)
    info = C.c_int64(0)
    f32 = torch.float32
    status = _lib.load().nq_op_cholesky_inverse(
        _ptr(G, "G", f32, 2), r, r, _ptr(L, "L", f32, 2), r, _ptr(Gi, "Ginv", f32, 2), r,
        C.byref(info), _stream(stream))
    if status not in (NQ_OK, _lib.NQ_ERR_NOT_POSITIVE_DEFINITE):
        _check(status, "nq_op_cholesky_inverse")
    return L, Gi, int(info.value)


def op_svid(X, T, stream=None):
    torch = _torch()
    rows, cols = X.shape
    f32 = torch.float32
    Z = torch.empty((rows, cols), dtype=f32, device=X.device)
    a = torch.empty((rows,), dtype=f32, device=X.device)
    b = torch.empty((cols,), dtype=f32, device=X.device)
    _check(_lib.load().nq_op_svid(_ptr(X, "X", f32, 2), rows, cols, cols, int(T),
                                  _ptr(Z, "Z", f32, 2), cols, _ptr(a, "a", f32, 1),
                                  _ptr(b, "b", f32, 1), _stream(stream)), "nq_op_svid")
    return Z, a, b


@dataclass
class Result:
    U: "object"
    V: "object"
    s1: "object"
    s2: "object"
    U_bits: "object"
    V_bits: "object"
    stats: Optional[dict]


class LBADMM:
    """One handle for one layer shape; reusable across runs of that shape."""

    def __init__(self, m, n, r, rho=1.0, iters=50, svid_steps=5, seed=0, compute_error=True,
                 init_exact=False, balance=True, single_stream=False, profile=False):
        """profile: False, True (every phase) or "rhs" (only the RHS GEMM)."""
        flags = 0
        flags |= NQ_FLAG_PROFILE if profile else 0
        flags |= NQ_FLAG_PROFILE_RHS_ONLY if profile == "rhs" else 0
        flags |= NQ_FLAG_COMPUTE_ERROR if compute_error else 0
        flags |= NQ_FLAG_INIT_EXACT if init_exact else 0
        flags |= 0 if balance else NQ_FLAG_NO_BALANCE
        flags |= NQ_FLAG_SINGLE_STREAM if single_stream else 0
        self.m, self.n, self.r = int(m), int(n), int(r)
        self.handle = lbadmm_create(m, n, r, rho, iters, svid_steps, seed, flags)

    def alloc_outputs(self, device):
        torch = _torch()
        nw = (self.r + 31) // 32
        f32 = torch.float32
        return dict(U=torch.empty((self.m, self.r), dtype=f32, device=device),
                    V=torch.empty((self.n, self.r), dtype=f32, device=device),
                    s1=torch.empty((self.m,), dtype=f32, device=device),
                    s2=torch.empty((self.n,), dtype=f32, device=device),
                    U_bits=torch.empty((self.m, nw), dtype=torch.int32, device=device),
                    V_bits=torch.empty((self.n, nw), dtype=torch.int32, device=device))

    def run(self, W, d_out, d_in, U0=None, V0=None, out=None, want_stats=True, stream=None):
        if out is None:
            out = self.alloc_outputs(W.device)
        st = lbadmm_run(self.handle, W, d_out, d_in, U0, V0, out["U"], out["V"], out["s1"],
                        out["s2"], out["U_bits"], out["V_bits"], want_stats, stream)
        return Result(out["U"], out["V"], out["s1"], out["s2"], out["U_bits"], out["V_bits"], st)

    def profile(self, reset=False):
        return lbadmm_profile(self.handle, reset)

    def state(self, stream=None):
        torch = _torch()
        f32 = torch.float32
        dev = torch.device("cuda", torch.cuda.current_device())
        s = {k: torch.empty((self.m if k in ("U", "Z_U", "Lam_U") else self.n, self.r),
                            dtype=f32, device=dev)
             for k in ("U", "V", "Z_U", "Lam_U", "Z_V", "Lam_V")}
        lbadmm_get_state(self.handle, stream=stream, **s)
        return s

    def close(self):
        if getattr(self, "handle", None):
            lbadmm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()


def lbadmm(W, d_out, d_in, r, rho=1.0, iters=50, svid_steps=5, U0=None, V0=None, seed=0,
           compute_error=True, init_exact=False, balance=True, single_stream=False) -> Result:
    """Factorise one layer: W ~ diag(s1) sign(U) sign(V)^T diag(s2)."""
    m, n = W.shape
    with LBADMM(m, n, r, rho, iters, svid_steps, seed, compute_error, init_exact, balance,
                single_stream) as h:
        return h.run(W, d_out, d_in, U0, V0)
