"""ctypes declarations of the C ABI in include/nq.h (argument marshalling only)."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnq.so")

NQ_OK = 0
NQ_ERR_INVALID_ARG = 1
NQ_ERR_UNSUPPORTED = 2
NQ_ERR_OUT_OF_MEMORY = 3
NQ_ERR_HIP = 4
NQ_ERR_NOT_POSITIVE_DEFINITE = 5
NQ_ERR_NONFINITE = 6
NQ_ERR_BAD_PRECONDITIONER = 7

NQ_FLAG_COMPUTE_ERROR = 0x1
NQ_FLAG_INIT_DRAWS = 0x2
NQ_FLAG_NO_BALANCE = 0x4
NQ_FLAG_SINGLE_STREAM = 0x8
NQ_FLAG_PROFILE = 0x10
NQ_FLAG_PROFILE_RHS_ONLY = 0x20
NQ_FLAG_SOLVE_CG = 0x40
NQ_FLAG_SOLVE_GD = 0x80

PHASES = ["gemm_rhs", "gemm_solve", "chain", "svid", "prep", "finish"]


class Desc(C.Structure):
    _fields_ = [("m", C.c_int64), ("n", C.c_int64), ("r", C.c_int64), ("rho", C.c_float),
                ("iters", C.c_int32), ("svid_steps", C.c_int32), ("seed", C.c_uint64),
                ("flags", C.c_uint32), ("solve_steps", C.c_int32)]


class Stats(C.Structure):
    _fields_ = [("rel_err_wtilde", C.c_double), ("rel_err_w", C.c_double),
                ("sumsq_wtilde", C.c_double), ("sigma0", C.c_double),
                ("potrf_info", C.c_int64), ("nonfinite", C.c_int32),
                ("bad_precond", C.c_int32), ("elapsed_ms", C.c_float),
                ("iters_done", C.c_int32), ("reserved", C.c_int32)]


P = C.c_void_p
I64 = C.c_int64
F32 = C.c_float
ST = C.c_int

# name -> (restype, argtypes); must match include/nq.h
SIGNATURES = {
    "nq_lbadmm_create": (ST, [C.POINTER(Desc), C.POINTER(P)]),
    "nq_lbadmm_workspace_bytes": (ST, [C.POINTER(Desc), C.POINTER(C.c_size_t)]),
    "nq_lbadmm_run": (ST, [P, P, I64, P, P, P, P, P, P, P, P, P, P, C.POINTER(Stats), P]),
    "nq_lbadmm_query": (ST, [P, C.POINTER(Stats)]),
    "nq_lbadmm_get_state": (ST, [P, P, P, P, P, P, P, P]),
    "nq_lbadmm_destroy": (None, [P]),
    "nq_lbadmm_profile": (ST, [P, C.POINTER(C.c_double), C.POINTER(I64), C.c_int32]),
    "nq_lbadmm_time_svid": (ST, [P, C.c_int32, C.c_int32, P, C.POINTER(C.c_double)]),
    "nq_pack_signs": (ST, [P, I64, I64, I64, P, I64, P]),
    "nq_transpose_signs": (ST, [P, I64, I64, I64, P, I64, P]),
    "nq_binary_matmul_work_floats": (I64, [I64, I64, I64]),
    "nq_binary_matmul": (ST, [P, I64, P, I64, I64, I64, I64, P, P, P, I64, I64, P, I64, P, P]),
    "nq_binary_matmul_noalloc": (ST, [P, I64, P, I64, I64, I64, I64, P, P, P, I64, I64, P, I64, P]),
    "nq_lw_create": (ST, [I64, I64, C.POINTER(P)]),
    "nq_lw_accumulate": (ST, [P, P, I64, I64, P]),
    "nq_lw_finalize": (ST, [P, P, C.POINTER(C.c_double), P]),
    "nq_lw_reset": (ST, [P]),
    "nq_lw_destroy": (ST, [P]),
    "nq_ste_create": (ST, [I64, I64, I64, I64, C.POINTER(P)]),
    "nq_ste_set_params": (ST, [P, P, P, P, P, P]),
    "nq_ste_step": (ST, [P, P, I64, P, I64, P, I64, C.c_float, P]),
    "nq_ste_last_loss": (ST, [P, C.POINTER(C.c_double), P]),
    "nq_ste_get_params": (ST, [P, P, P, P, P, P]),
    "nq_ste_destroy": (ST, [P]),
    "nq_op_precondition": (ST, [P, I64, I64, I64, P, P, P, I64, P]),
    "nq_op_gram": (ST, [P, I64, I64, I64, F32, P, I64, P]),
    "nq_op_gemm_rhs": (ST, [P, I64, P, I64, P, I64, F32, P, I64, I64, I64, I64, P]),
    "nq_op_sign_gemm": (ST, [P, I64, P, I64, P, I64, P, I64, I64, I64, I64, P]),
    "nq_op_cholesky_inverse": (ST, [P, I64, I64, P, I64, P, I64, C.POINTER(I64), P]),
    "nq_op_svid": (ST, [P, I64, I64, I64, C.c_int32, P, I64, P, P, P]),
    "nq_op_svid_dual": (ST, [P, P, I64, I64, I64, C.c_int32, P, P, I64, P, P, P]),
    "nq_status_string": (C.c_char_p, [ST]),
    "nq_last_error_message": (C.c_char_p, []),
    "nq_version": (C.c_int32, []),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libnq.so once. torch is imported first so that the process holds a
    single HIP runtime (libnq.so resolves libamdhip64.so.7 to torch's copy)."""
    global _lib
    if _lib is not None:
        return _lib
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - torch is part of the image
        pass
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sub_bit_weight_lb_amd.build` "
                          "or __graft_entry__.build()")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
