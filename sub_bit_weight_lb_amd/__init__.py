"""LB-ADMM low-rank binary factorisation on MI355X (gfx950).

Thin Python binding of the C ABI in include/nq.h. Every step of the
per-layer path runs in the HIP kernels of libnq.so; this module only checks
and marshals arguments (torch tensors supply device memory and the current
stream). Importing works without a GPU; calls that need the device fail
loudly when libnq.so or the GPU is missing. There is no CPU fallback.

Functions mirror the C names without the ``nq_`` prefix:
    lbadmm_create / lbadmm_run / lbadmm_query / lbadmm_get_state /
    lbadmm_destroy / lbadmm_workspace_bytes / pack_signs /
    transpose_signs / binary_matmul / binary_matmul_noalloc / lw_* (LedoitWolf) /
    ste_* (STERefiner) /
    op_precondition / op_gram / op_gemm_rhs / op_cholesky_inverse / op_svid
plus the conveniences ``LBADMM`` (a handle object) and ``lbadmm`` (one call).
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional

from . import _lib
from ._lib import (NQ_FLAG_COMPUTE_ERROR, NQ_FLAG_INIT_DRAWS, NQ_FLAG_NO_BALANCE,  # noqa: F401
                   NQ_FLAG_PROFILE, NQ_FLAG_PROFILE_RHS_ONLY, NQ_FLAG_SINGLE_STREAM,
                   NQ_FLAG_SOLVE_CG, NQ_FLAG_SOLVE_GD, NQ_OK, PHASES, Desc, Stats)

__all__ = [
    "NQError", "lbadmm_create", "lbadmm_run", "lbadmm_query", "lbadmm_get_state",
    "lbadmm_destroy", "lbadmm_profile", "lbadmm_workspace_bytes", "pack_signs", "transpose_signs",
    "binary_matmul", "binary_matmul_noalloc", "binary_matmul_work_floats", "LedoitWolf", "ledoit_wolf_diag",
    "preconditioners", "STERefiner", "cosine_lr", "op_precondition", "op_gram",
    "op_gemm_rhs", "op_sign_gemm", "op_cholesky_inverse", "op_svid", "LBADMM", "lbadmm", "Result",
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


def _desc(m, n, r, rho, iters, svid_steps, seed, flags, solve_steps=0) -> Desc:
    return Desc(int(m), int(n), int(r), float(rho), int(iters), int(svid_steps), int(seed),
                int(flags), int(solve_steps))


def lbadmm_workspace_bytes(m, n, r, rho=1.0, iters=50, svid_steps=5, seed=0, flags=0,
                           solve_steps=0) -> int:
    out = C.c_size_t(0)
    d = _desc(m, n, r, rho, iters, svid_steps, seed, flags, solve_steps)
    _check(_lib.load().nq_lbadmm_workspace_bytes(C.byref(d), C.byref(out)),
           "nq_lbadmm_workspace_bytes")
    return int(out.value)


def lbadmm_create(m, n, r, rho=1.0, iters=50, svid_steps=5, seed=0,
                  flags=NQ_FLAG_COMPUTE_ERROR, solve_steps=0) -> int:
    h = C.c_void_p(0)
    d = _desc(m, n, r, rho, iters, svid_steps, seed, flags, solve_steps)
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


def lbadmm_time_svid(h, factor, reps=10, stream=None) -> float:
    """Average device ms of one SVID + dual update of factor 0 (U) or 1 (V),
    `reps` back to back on the handle's state after a run."""
    ms = C.c_double()
    _check(_lib.load().nq_lbadmm_time_svid(C.c_void_p(h), int(factor), int(reps), _stream(stream),
                                           C.byref(ms)), "nq_lbadmm_time_svid")
    return float(ms.value)


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
    if bits.shape[1] < (cols + 31) // 32:
        raise ValueError(f"bits has {bits.shape[1]} words per row, needs ceil(cols/32)")
    if out is None:
        out = torch.empty((cols, (rows + 31) // 32), dtype=torch.int32, device=bits.device)
    elif (out.dim() != 2 or out.stride(1) != 1 or out.shape[0] < cols
          or out.shape[1] < (rows + 31) // 32):
        raise ValueError(f"out must be 2-D with unit column stride and at least {cols} x "
                         f"{(rows + 31) // 32} words, got {tuple(out.shape)}")
    _check(_lib.load().nq_transpose_signs(
        _ptr(bits, "bits", torch.int32, 2, need_contig=False), rows, cols, bits.stride(0),
        _ptr(out, "out", torch.int32, 2, need_contig=False), out.stride(0), _stream(stream)),
        "nq_transpose_signs")
    return out


def binary_matmul_work_floats(B, n, r):
    """Floats of workspace binary_matmul needs for B inputs of width n and
    rank r: the formula of nq_binary_matmul_work_floats (8 partial sums per
    input and rank, rounded up to 64 floats, then the inputs' bf16 terms,
    3072 floats per 16 inputs and 128 columns of the wider product),
    computed here so that buffer checks need no library call."""
    B, n, r = int(B), int(n), int(r)
    if B < 0 or n < 0 or r < 0:
        return -1
    return -(-8 * B * r // 64) * 64 + 3072 * (-(-B // 16)) * (-(-max(n, r) // 128))


def binary_matmul(U_bits, Vt_bits, s1, s2, X, r, Y=None, work=None, stream=None):
    """Y = X W^T for the factorised layer W = diag(s1) S_U S_V^T diag(s2):
    U_bits (m x ceil(r/32) int32), Vt_bits (r x ceil(n/32) int32, from
    transpose_signs of the run's V_bits), s1 (m), s2 (n), X (B x n float32,
    or a vector of length n); work, if given, holds
    binary_matmul_work_floats(B, n, r) float32 (16-byte aligned). Returns Y
    (B x m, or length m)."""
    torch = _torch()
    vec = X.dim() == 1
    X2 = X.unsqueeze(0) if vec else X
    if X2.dim() != 2 or X2.stride(1) != 1:
        raise ValueError("X must be 1-D or 2-D with unit column stride")
    B, n = X2.shape
    m = _check_binmm_shapes(U_bits, Vt_bits, s1, s2, n, r)
    Y2 = _binmm_out(Y, B, m, vec, X.device)
    need = binary_matmul_work_floats(B, n, r)
    if work is None:
        work = torch.empty((max(need, 1),), dtype=torch.float32, device=X.device)
    elif work.numel() < need:
        raise ValueError(f"work holds {work.numel()} floats, needs {need}")
    elif work.data_ptr() % 16:
        raise ValueError("work must be 16-byte aligned")
    _check(_lib.load().nq_binary_matmul(
        _ptr(U_bits, "U_bits", torch.int32, 2, need_contig=False), U_bits.stride(0),
        _ptr(Vt_bits, "Vt_bits", torch.int32, 2, need_contig=False), Vt_bits.stride(0),
        m, n, r, _ptr(s1, "s1", torch.float32), _ptr(s2, "s2", torch.float32),
        _ptr(X2, "X", torch.float32, 2, need_contig=False), B, X2.stride(0),
        _ptr(Y2, "Y", torch.float32, 2, need_contig=False), Y2.stride(0),
        _ptr(work, "work", torch.float32), _stream(stream)), "nq_binary_matmul")
    return Y2[0] if vec else Y2


# Workspace limit of binary_matmul_noalloc: its fixed scratch holds 2^23
# floats, so binary_matmul_work_floats(B, n, r) must not exceed that
NOALLOC_MAX_FLOATS = 1 << 23


def binary_matmul_noalloc(U_bits, Vt_bits, s1, s2, X, r, Y, stream=None):
    """binary_matmul into a caller-given Y with no device allocation: the
    library's fixed per-GPU scratch is the workspace, so
    binary_matmul_work_floats(B, n, r) must not exceed NOALLOC_MAX_FLOATS.
    Calls that overlap on one GPU race; calls ordered on one stream do not.
    Returns Y."""
    torch = _torch()
    vec = X.dim() == 1
    X2 = X.unsqueeze(0) if vec else X
    if X2.dim() != 2 or X2.stride(1) != 1:
        raise ValueError("X must be 1-D or 2-D with unit column stride")
    B, n = X2.shape
    m = _check_binmm_shapes(U_bits, Vt_bits, s1, s2, n, r)
    if Y is None:
        raise ValueError("Y is required: this entry point allocates nothing")
    Y2 = _binmm_out(Y, B, m, vec, X.device)
    need = binary_matmul_work_floats(B, n, r)
    if need > NOALLOC_MAX_FLOATS:
        raise ValueError(f"the call needs {need} floats of workspace, more than the fixed "
                         f"scratch ({NOALLOC_MAX_FLOATS})")
    _check(_lib.load().nq_binary_matmul_noalloc(
        _ptr(U_bits, "U_bits", torch.int32, 2, need_contig=False), U_bits.stride(0),
        _ptr(Vt_bits, "Vt_bits", torch.int32, 2, need_contig=False), Vt_bits.stride(0),
        m, n, r, _ptr(s1, "s1", torch.float32), _ptr(s2, "s2", torch.float32),
        _ptr(X2, "X", torch.float32, 2, need_contig=False), B, X2.stride(0),
        _ptr(Y2, "Y", torch.float32, 2, need_contig=False), Y2.stride(0), _stream(stream)),
        "nq_binary_matmul_noalloc")
    return Y


def _check_binmm_shapes(U_bits, Vt_bits, s1, s2, n, r):
    """Checks the factor operands of the binary-layer product against n and r
    (the C ABI cannot see buffer sizes); returns m."""
    for t, name in ((U_bits, "U_bits"), (Vt_bits, "Vt_bits")):
        if t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be 2-D with unit column stride")
    m = U_bits.shape[0]
    if U_bits.shape[1] < (r + 31) // 32:
        raise ValueError(f"U_bits has {U_bits.shape[1]} words per row, needs ceil(r/32)")
    if Vt_bits.shape[0] != r or Vt_bits.shape[1] < (n + 31) // 32:
        raise ValueError(f"Vt_bits must be r x (>= ceil(n/32)) words, got {tuple(Vt_bits.shape)}")
    if s1.numel() != m or s2.numel() != n:
        raise ValueError("s1 must hold m and s2 n values")
    return m


def _binmm_out(Y, B, m, vec, device):
    """Y as a B x m view with unit column stride (a vector when X is one),
    allocated when None."""
    torch = _torch()
    if Y is None:
        return torch.empty((B, m), dtype=torch.float32, device=device)
    Y2 = Y.unsqueeze(0) if (vec and Y.dim() == 1) else Y
    if Y2.dim() != 2 or Y2.stride(1) != 1 or Y2.shape[0] < B or Y2.shape[1] < m:
        raise ValueError(f"Y must be 2-D with unit column stride and at least {B} x {m}, "
                         f"got {tuple(Y.shape)}")
    return Y2


class LedoitWolf:
    """Running Ledoit-Wolf statistics of activation samples with p features
    (nq_lw_*): accumulate() chunks of tokens x p float32 samples, then
    finalize() -> (d, shrinkage), d the diagonal of the preconditioner
    sqrt(diag(shrunk second moment)) as a float32 device vector."""

    def __init__(self, p, max_rows=16384):
        h = C.c_void_p(0)
        _check(_lib.load().nq_lw_create(int(p), int(max_rows), C.byref(h)), "nq_lw_create")
        self.handle, self.p = h.value, int(p)

    def accumulate(self, Z, stream=None):
        torch = _torch()
        if Z.dim() != 2 or Z.shape[1] != self.p or Z.stride(1) != 1:
            raise ValueError(f"Z must be rows x {self.p} with unit column stride")
        _check(_lib.load().nq_lw_accumulate(
            C.c_void_p(self.handle), _ptr(Z, "Z", torch.float32, 2, need_contig=False),
            Z.shape[0], Z.stride(0), _stream(stream)), "nq_lw_accumulate")

    def finalize(self, d=None, stream=None):
        torch = _torch()
        if d is None:
            dev = torch.device("cuda", torch.cuda.current_device())
            d = torch.empty(self.p, dtype=torch.float32, device=dev)
        elif d.numel() != self.p:
            raise ValueError(f"d must hold {self.p} values")
        shrink = C.c_double(0.0)
        _check(_lib.load().nq_lw_finalize(C.c_void_p(self.handle), _ptr(d, "d", torch.float32),
                                          C.byref(shrink), _stream(stream)), "nq_lw_finalize")
        return d, shrink.value

    def reset(self):
        _check(_lib.load().nq_lw_reset(C.c_void_p(self.handle)), "nq_lw_reset")

    def close(self):
        if getattr(self, "handle", None):
            _lib.load().nq_lw_destroy(C.c_void_p(self.handle))
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def ledoit_wolf_diag(Z, max_rows=16384, stream=None):
    """(d, shrinkage) for one sample matrix Z (device, tokens x p float32)."""
    with LedoitWolf(Z.shape[1], min(max_rows, max(1, Z.shape[0]))) as lw:
        lw.accumulate(Z, stream)
        return lw.finalize(stream=stream)


def preconditioners(X_in, Z_out, max_rows=16384, stream=None):
    """(d_out, d_in) of a layer from its input-side sample X_in (N x n) and
    output-side sample Z_out (N x m), ready for nq_lbadmm_run."""
    d_in, _ = ledoit_wolf_diag(X_in, max_rows, stream)
    d_out, _ = ledoit_wolf_diag(Z_out, max_rows, stream)
    return d_out, d_in


def cosine_lr(t, K, lr_max=1e-4, lr_min=1e-6):
    """Learning rate of step t (0-based) of K on the cosine schedule."""
    import math
    return lr_min + (lr_max - lr_min) * (1.0 + math.cos(math.pi * t / K)) / 2.0


class STERefiner:
    """STE refinement of one factorised layer (nq_ste_*): set_params() from
    a run's U, V, s1, s2, then step() per batch (X, Y = X W^T device float32;
    rows: an int32 device index vector or None), or refine() over a list of
    batches with the cosine schedule."""

    def __init__(self, m, n, r, max_tokens):
        h = C.c_void_p(0)
        _check(_lib.load().nq_ste_create(int(m), int(n), int(r), int(max_tokens), C.byref(h)),
               "nq_ste_create")
        self.handle, self.m, self.n, self.r = h.value, int(m), int(n), int(r)
        self.max_tokens = int(max_tokens)

    def set_params(self, U, V, s1, s2, stream=None):
        torch = _torch()
        f32 = torch.float32
        if (tuple(U.shape) != (self.m, self.r) or tuple(V.shape) != (self.n, self.r)
                or s1.numel() != self.m or s2.numel() != self.n):
            raise ValueError("U, V, s1, s2 must be m x r, n x r, m and n")
        _check(_lib.load().nq_ste_set_params(
            C.c_void_p(self.handle), _ptr(U, "U", f32, 2), _ptr(V, "V", f32, 2),
            _ptr(s1, "s1", f32), _ptr(s2, "s2", f32), _stream(stream)), "nq_ste_set_params")

    def step(self, X, Y, lr, rows=None, stream=None, check_rows=True):
        """check_rows: verify on the host that every index is a row of X
        (a device read and a wait; the library cannot see X's length)."""
        torch = _torch()
        f32 = torch.float32
        if X.dim() != 2 or X.shape[1] != self.n or X.stride(1) != 1:
            raise ValueError(f"X must be tokens x {self.n} with unit column stride")
        if Y.dim() != 2 or Y.shape[1] != self.m or Y.stride(1) != 1 or Y.shape[0] != X.shape[0]:
            raise ValueError(f"Y must be tokens x {self.m}, as many rows as X")
        if rows is None:
            T = X.shape[0]
            rp = None
        else:
            if rows.dtype != torch.int32 or rows.dim() != 1:
                raise ValueError("rows must be a 1-D int32 tensor")
            T = rows.numel()
            rp = _ptr(rows, "rows", torch.int32)
            if check_rows and T and (int(rows.min()) < 0 or int(rows.max()) >= X.shape[0]):
                raise ValueError("rows holds an index outside X")
        if not 1 <= T <= self.max_tokens:
            raise ValueError(f"a batch holds 1 .. {self.max_tokens} tokens")
        _check(_lib.load().nq_ste_step(
            C.c_void_p(self.handle), _ptr(X, "X", f32, 2, need_contig=False), X.stride(0),
            _ptr(Y, "Y", f32, 2, need_contig=False), Y.stride(0), rp, T, float(lr),
            _stream(stream)), "nq_ste_step")

    def last_loss(self, stream=None):
        out = C.c_double(0.0)
        _check(_lib.load().nq_ste_last_loss(C.c_void_p(self.handle), C.byref(out),
                                            _stream(stream)), "nq_ste_last_loss")
        return out.value

    def params(self, stream=None):
        torch = _torch()
        dev = torch.device("cuda", torch.cuda.current_device())
        f32 = torch.float32
        U = torch.empty((self.m, self.r), dtype=f32, device=dev)
        V = torch.empty((self.n, self.r), dtype=f32, device=dev)
        s1 = torch.empty(self.m, dtype=f32, device=dev)
        s2 = torch.empty(self.n, dtype=f32, device=dev)
        _check(_lib.load().nq_ste_get_params(
            C.c_void_p(self.handle), _ptr(U, "U", f32), _ptr(V, "V", f32), _ptr(s1, "s1", f32),
            _ptr(s2, "s2", f32), _stream(stream)), "nq_ste_get_params")
        return U, V, s1, s2

    def refine(self, X, Y, batches, lr_max=1e-4, lr_min=1e-6, losses=True, stream=None,
               check_rows=True):
        """One step per batch (int32 device index vectors) on the cosine
        schedule from lr_max to lr_min; returns the per-step losses (each
        read back, which waits for the stream) or None."""
        out = [] if losses else None
        K = len(batches)
        for t, rows in enumerate(batches):
            self.step(X, Y, cosine_lr(t, K, lr_max, lr_min), rows, stream, check_rows)
            if losses:
                out.append(self.last_loss(stream))
        return out

    def close(self):
        if getattr(self, "handle", None):
            _lib.load().nq_ste_destroy(C.c_void_p(self.handle))
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


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


def op_sign_gemm(A, S, transposed=False, stream=None):
    """C = A S^T for A (rows x k) and a +-1 matrix S (cols x k), on the bf16
    matrix cores; with transposed=True returns (C, C^T from the kernel)."""
    torch = _torch()
    rows, k = A.shape
    cols, k2 = S.shape
    if k2 != k:
        raise ValueError("A and S must have the same number of columns")
    f32 = torch.float32
    Cm = torch.empty((rows, cols), dtype=f32, device=A.device)
    Ct = torch.empty((cols, rows), dtype=f32, device=A.device) if transposed else None
    _check(_lib.load().nq_op_sign_gemm(
        _ptr(A, "A", f32, 2), k, _ptr(S, "S", f32, 2), k, _ptr(Cm, "C", f32, 2), cols,
        _ptr(Ct, "Ct", f32, 2, True), rows, rows, cols, k, _stream(stream)), "nq_op_sign_gemm")
    return (Cm, Ct) if transposed else Cm


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


def op_svid_dual(U, Lam, T, stream=None):
    """X = U + Lam, Z = SVID_T(X), Lam_out = X - Z: returns (Z, Lam_out, a, b)."""
    torch = _torch()
    rows, cols = U.shape
    if tuple(Lam.shape) != (rows, cols):
        raise ValueError("U and Lam must have the same shape")
    f32 = torch.float32
    Z = torch.empty((rows, cols), dtype=f32, device=U.device)
    Lo = torch.empty((rows, cols), dtype=f32, device=U.device)
    a = torch.empty((rows,), dtype=f32, device=U.device)
    b = torch.empty((cols,), dtype=f32, device=U.device)
    _check(_lib.load().nq_op_svid_dual(_ptr(U, "U", f32, 2), _ptr(Lam, "Lam", f32, 2), rows, cols,
                                       cols, int(T), _ptr(Z, "Z", f32, 2), _ptr(Lo, "Lam_out", f32, 2),
                                       cols, _ptr(a, "a", f32, 1), _ptr(b, "b", f32, 1),
                                       _stream(stream)), "nq_op_svid_dual")
    return Z, Lo, a, b


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
                 init_draws=False, balance=True, single_stream=False, profile=False,
                 solver=None):
        """init_draws: U0/V0 passed to run() are standard-normal draws that
        the run scales by sigma0 (default: they are the starting latents).
        profile: False, True (every phase) or "rhs" (only the RHS GEMM).
        solver: None (the Cholesky solve) or (method, steps) with method "cg"
        (conjugate gradients) or "gd" (steepest descent): an iterative solve
        of each half's system, warm-started from the factor's previous value."""
        flags, steps = 0, 0
        if solver is not None:
            method, steps = solver
            if method not in ("cg", "gd"):
                raise ValueError("solver method is 'cg' or 'gd'")
            flags |= NQ_FLAG_SOLVE_CG if method == "cg" else NQ_FLAG_SOLVE_GD
        flags |= NQ_FLAG_PROFILE if profile else 0
        flags |= NQ_FLAG_PROFILE_RHS_ONLY if profile == "rhs" else 0
        flags |= NQ_FLAG_COMPUTE_ERROR if compute_error else 0
        flags |= NQ_FLAG_INIT_DRAWS if init_draws else 0
        flags |= 0 if balance else NQ_FLAG_NO_BALANCE
        flags |= NQ_FLAG_SINGLE_STREAM if single_stream else 0
        self.m, self.n, self.r = int(m), int(n), int(r)
        self.handle = lbadmm_create(m, n, r, rho, iters, svid_steps, seed, flags, steps)

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

    def time_svid(self, factor, reps=10, stream=None):
        return lbadmm_time_svid(self.handle, factor, reps, stream)

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
           compute_error=True, init_draws=False, balance=True, single_stream=False,
           solver=None) -> Result:
    """Factorise one layer: W ~ diag(s1) sign(U) sign(V)^T diag(s2)."""
    m, n = W.shape
    with LBADMM(m, n, r, rho, iters, svid_steps, seed, compute_error, init_draws, balance,
                single_stream, solver=solver) as h:
        return h.run(W, d_out, d_in, U0, V0)
