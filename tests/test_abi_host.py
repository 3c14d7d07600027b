"""Host-side checks of the C ABI (no GPU needed, no compute calls)."""
import ctypes as C
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nq.h")

from sub_bit_weight_lb_amd import _lib as L  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nq_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libnq.so is not built; run __graft_entry__.build() first")
    return L.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    # and the binding declares a signature for each of them
    assert set(names) == set(L.SIGNATURES), set(names) ^ set(L.SIGNATURES)


def test_struct_layouts_match_header(tmp_path):
    src = tmp_path / "sz.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "nq.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu %zu\\n\", sizeof(nq_lbadmm_desc),"
        " offsetof(nq_lbadmm_desc, seed), offsetof(nq_lbadmm_desc, flags),"
        " offsetof(nq_lbadmm_desc, solve_steps),"
        " sizeof(nq_lbadmm_stats), offsetof(nq_lbadmm_stats, potrf_info),"
        " offsetof(nq_lbadmm_stats, elapsed_ms)); return 0;}\n")
    exe = tmp_path / "sz"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src),
                           "-o", str(exe)])
    vals = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    assert vals == [C.sizeof(L.Desc), L.Desc.seed.offset, L.Desc.flags.offset,
                    L.Desc.solve_steps.offset,
                    C.sizeof(L.Stats), L.Stats.potrf_info.offset, L.Stats.elapsed_ms.offset]


def test_status_strings_and_version(lib):
    for code in range(8):
        assert lib.nq_status_string(code).decode().startswith("NQ_")
    assert lib.nq_status_string(99).decode() == "NQ_ERR_UNKNOWN"
    assert lib.nq_version() >= 100


def _desc(**kw):
    d = dict(m=256, n=512, r=128, rho=1.0, iters=2, svid_steps=5, seed=0, flags=0, solve_steps=0)
    d.update(kw)
    return L.Desc(**d)


@pytest.mark.parametrize("bad", [dict(m=0), dict(n=-1), dict(r=0), dict(rho=0.0),
                                 dict(rho=float("nan")), dict(rho=float("inf")), dict(iters=-1),
                                 dict(svid_steps=0), dict(flags=0x100), dict(r=1 << 17),
                                 dict(flags=0xC0, solve_steps=3), dict(flags=0x40),
                                 dict(flags=0x80, solve_steps=10001), dict(solve_steps=2),
                                 dict(r=(1 << 13) + 1), dict(m=(1 << 21) - 255),
                                 dict(n=(1 << 21) - 255)])
def test_create_rejects_bad_desc_before_device_work(lib, bad):
    h = C.c_void_p(0)
    st = lib.nq_lbadmm_create(C.byref(_desc(**bad)), C.byref(h))
    assert st == L.NQ_ERR_INVALID_ARG
    assert h.value is None
    assert lib.nq_last_error_message().decode()
    sz = C.c_size_t(0)
    assert lib.nq_lbadmm_workspace_bytes(C.byref(_desc(**bad)), C.byref(sz)) == L.NQ_ERR_INVALID_ARG


def test_desc_limits_accept_the_largest_shapes(lib):
    # padded m, n below 2^21 (32-bit row offsets of the tiled products) and
    # r <= 2^13 (the SVID's per-workgroup column blocks) are sized, not refused
    sz = C.c_size_t(0)
    assert lib.nq_lbadmm_workspace_bytes(
        C.byref(_desc(m=(1 << 21) - 256, n=256, r=128)), C.byref(sz)) == 0
    assert lib.nq_lbadmm_workspace_bytes(C.byref(_desc(r=1 << 13)), C.byref(sz)) == 0


def test_time_svid_rejects_bad_arguments(lib):
    ms = C.c_double(0.0)
    assert lib.nq_lbadmm_time_svid(None, 0, 1, None, C.byref(ms)) == L.NQ_ERR_INVALID_ARG


def test_create_null_arguments(lib):
    assert lib.nq_lbadmm_create(None, None) == L.NQ_ERR_INVALID_ARG
    h = C.c_void_p(0)
    assert lib.nq_lbadmm_create(None, C.byref(h)) == L.NQ_ERR_INVALID_ARG


def test_workspace_bytes_accounts_for_padding(lib):
    def ws(**kw):
        s = C.c_size_t(0)
        assert lib.nq_lbadmm_workspace_bytes(C.byref(_desc(**kw)), C.byref(s)) == 0
        return s.value
    a = ws(m=256, n=512, r=128)
    # same padded shapes -> same bytes; bigger shapes -> more
    assert ws(m=250, n=500, r=100) == a
    assert ws(m=4096, n=4096, r=2048) > 32 * a
    # config-sized layer stays far below 288 GB of HBM
    big = ws(m=8192, n=28672, r=6144)
    assert 4e9 < big < 20e9


@pytest.mark.skipif(os.environ.get("HIP_VISIBLE_DEVICES") is None and
                    os.path.exists("/dev/kfd"), reason="a GPU may be visible")
def test_create_without_device_reports_unsupported(lib):
    h = C.c_void_p(0)
    st = lib.nq_lbadmm_create(C.byref(_desc()), C.byref(h))
    assert st in (L.NQ_ERR_UNSUPPORTED, L.NQ_ERR_HIP)
    assert h.value is None


def test_run_and_query_reject_null_handle(lib):
    assert lib.nq_lbadmm_run(None, None, 0, None, None, None, None, None, None, None, None,
                             None, None, None, None) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_lbadmm_query(None, None) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_lbadmm_get_state(None, None, None, None, None, None, None, None) == \
        L.NQ_ERR_INVALID_ARG
    lib.nq_lbadmm_destroy(None)


def test_pack_signs_argument_checks(lib):
    assert lib.nq_pack_signs(None, 0, 5, 5, None, 1, None) == 0          # empty is a no-op
    assert lib.nq_pack_signs(None, 3, 0, 0, None, 0, None) == 0
    assert lib.nq_pack_signs(None, 3, 5, 5, None, 1, None) == L.NQ_ERR_INVALID_ARG
    fake = C.c_void_p(0x1000)
    assert lib.nq_pack_signs(fake, 3, 40, 39, fake, 2, None) == L.NQ_ERR_INVALID_ARG  # ldx < cols
    assert lib.nq_pack_signs(fake, 3, 40, 40, fake, 1, None) == L.NQ_ERR_INVALID_ARG  # words
    assert lib.nq_pack_signs(fake, -1, 40, 40, fake, 2, None) == L.NQ_ERR_INVALID_ARG


def test_binary_layer_argument_checks(lib):
    f = C.c_void_p(0x1000)
    # transpose: empty is a no-op; strides below the packed widths are rejected
    assert lib.nq_transpose_signs(None, 0, 5, 1, None, 1, None) == 0
    assert lib.nq_transpose_signs(f, 40, 70, 2, f, 2, None) == L.NQ_ERR_INVALID_ARG   # ld_in < 3
    assert lib.nq_transpose_signs(f, 40, 70, 3, f, 1, None) == L.NQ_ERR_INVALID_ARG   # ld_out < 2
    assert lib.nq_transpose_signs(None, 4, 4, 1, f, 1, None) == L.NQ_ERR_INVALID_ARG
    # matmul: m == 0 or B == 0 is a no-op
    args = dict(ldu=2, ldvt=3, m=10, n=70, r=40, B=2, ldx=70, ldy=10)

    def call(work=f, **kw):
        a = dict(args, **kw)
        return lib.nq_binary_matmul(f, a["ldu"], f, a["ldvt"], a["m"], a["n"], a["r"], f, f, f,
                                    a["B"], a["ldx"], f, a["ldy"], work, None)
    assert call(m=0) == 0 and call(B=0) == 0
    assert call(work=None) == L.NQ_ERR_INVALID_ARG
    assert call(work=C.c_void_p(0x1004)) == L.NQ_ERR_INVALID_ARG   # not 16-byte aligned
    assert call(ldu=1) == L.NQ_ERR_INVALID_ARG          # < ceil(40/32)
    assert call(ldvt=2) == L.NQ_ERR_INVALID_ARG         # < ceil(70/32)
    assert call(ldx=69) == L.NQ_ERR_INVALID_ARG
    assert call(ldy=9) == L.NQ_ERR_INVALID_ARG
    assert call(r=0) == L.NQ_ERR_INVALID_ARG
    assert call(n=-1) == L.NQ_ERR_INVALID_ARG

    # the workspace size: 8 B r partial sums (rounded up to 64 floats), then
    # the bf16 terms, 3072 floats per 16 inputs and 128 columns of the wider
    # of the two products
    ws = lib.nq_binary_matmul_work_floats
    assert ws(2, 70, 40) == 640 + 3072
    assert ws(16, 28672, 6144) == 8 * 16 * 6144 + 3072 * 224
    assert ws(17, 100, 300) == 40832 + 3072 * 2 * 3   # 8 * 17 * 300 = 40800, rounded up to 64
    assert ws(1, 1, 1) == 64 + 3072
    assert ws(-1, 4, 4) == -1
    # the binding's copy of the formula (it checks buffers without calling
    # the library) agrees with the library's
    import sub_bit_weight_lb_amd as nq
    for B, n, r in ((1, 1, 1), (2, 70, 40), (9, 4100, 2049), (33, 1000, 33), (128, 2048, 6656),
                    (16, 28672, 6144), (0, 5, 5), (3, 0, 7)):
        assert nq.binary_matmul_work_floats(B, n, r) == ws(B, n, r), (B, n, r)

    # the fixed-scratch variant: the same checks, and the workspace must fit
    # its 2^23 floats
    def call_na(**kw):
        a = dict(args, **kw)
        return lib.nq_binary_matmul_noalloc(f, a["ldu"], f, a["ldvt"], a["m"], a["n"], a["r"],
                                            f, f, f, a["B"], a["ldx"], f, a["ldy"], None)
    assert call_na(m=0) == 0 and call_na(B=0) == 0
    assert call_na(ldu=1) == L.NQ_ERR_INVALID_ARG
    assert call_na(ldy=9) == L.NQ_ERR_INVALID_ARG
    assert ws(129, 70, 8192) > 1 << 23
    assert call_na(r=8192, ldu=256, B=129) == L.NQ_ERR_INVALID_ARG
    assert ws(2, 1 << 22, 40) > 1 << 23
    assert call_na(n=1 << 22, ldvt=1 << 17, ldx=1 << 22) == L.NQ_ERR_INVALID_ARG


def test_ledoit_wolf_argument_checks(lib):
    h = C.c_void_p(0)
    assert lib.nq_lw_create(0, 16, C.byref(h)) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_lw_create(16385, 16, C.byref(h)) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_lw_create(8, 0, C.byref(h)) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_lw_create(8, (1 << 20) + 1, C.byref(h)) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_lw_create(16384, 1 << 17, C.byref(h)) == L.NQ_ERR_INVALID_ARG  # > 2^30 staged
    assert h.value is None
    f = C.c_void_p(0x1000)
    d = C.c_double(0)
    assert lib.nq_lw_accumulate(None, f, 4, 8, None) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_lw_finalize(None, f, C.byref(d), None) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_lw_reset(None) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_lw_destroy(None) == 0


def test_ops_argument_checks(lib):
    f = C.c_void_p(0x1000)
    info = C.c_int64(0)
    assert lib.nq_op_precondition(f, 3, 4, 5, f, f, f, 5, None) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_op_gram(f, 0, 4, 4, 1.0, f, 4, None) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_op_gemm_rhs(f, 2, f, 4, None, 0, 1.0, f, 4, 3, 4, 5, None) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_op_cholesky_inverse(f, 4, 3, f, 4, f, 4, C.byref(info), None) == \
        L.NQ_ERR_INVALID_ARG
    assert lib.nq_op_svid(f, 4, 4, 4, 0, f, 4, None, None, None) == L.NQ_ERR_INVALID_ARG
    # sign gemm: lda < k, lds < k, ldc < cols, ldct < rows, a missing operand
    assert lib.nq_op_sign_gemm(f, 4, f, 5, f, 6, None, 0, 3, 6, 5, None) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_op_sign_gemm(f, 5, f, 4, f, 6, None, 0, 3, 6, 5, None) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_op_sign_gemm(f, 5, f, 5, f, 5, None, 0, 3, 6, 5, None) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_op_sign_gemm(f, 5, f, 5, f, 6, f, 2, 3, 6, 5, None) == L.NQ_ERR_INVALID_ARG
    assert lib.nq_op_sign_gemm(None, 5, f, 5, f, 6, None, 0, 3, 6, 5, None) == L.NQ_ERR_INVALID_ARG


def test_binding_imports_and_missing_library_fails_loudly(tmp_path):
    code = ("import sub_bit_weight_lb_amd._lib as L\n"
            "try:\n    L.load('%s')\nexcept ImportError as e:\n    print('IMPORTERROR', e)\n"
            % str(tmp_path / "nope.so"))
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert "IMPORTERROR" in out.stdout, out.stderr


def test_product_package_never_imports_oracle():
    pkg = os.path.join(ROOT, "sub_bit_weight_lb_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt.replace("oracle is", ""), f
