"""The Python binding is the only place that sees buffer sizes (the C ABI
takes pointers), so a short output or scratch buffer must be refused there,
before any call into the library. These run on the CPU: the library loader
is replaced by one that fails, so a check that let a call through would show
up as that failure rather than a ValueError."""
import pytest
import torch

import sub_bit_weight_lb_amd as nq
from sub_bit_weight_lb_amd import _lib


@pytest.fixture
def no_library(monkeypatch):
    def boom():
        raise AssertionError("the library was called")
    monkeypatch.setattr(_lib, "load", boom)


def operands(m=40, n=70, r=33, B=3):
    i32 = torch.int32
    return dict(U_bits=torch.zeros((m, (r + 31) // 32), dtype=i32),
                Vt_bits=torch.zeros((r, (n + 31) // 32), dtype=i32),
                s1=torch.ones(m), s2=torch.ones(n), X=torch.zeros((B, n)), r=r)


@pytest.mark.parametrize("change, what", [
    (dict(work=torch.zeros(nq.binary_matmul_work_floats(3, 70, 33) - 1)), "work"),
    (dict(Y=torch.zeros((2, 40))), "Y"),
    (dict(Y=torch.zeros((3, 39))), "Y"),
    (dict(Y=torch.zeros((3, 80))[:, ::2]), "Y"),     # column stride 2
    (dict(U_bits=torch.zeros((40, 1), dtype=torch.int32)), "U_bits"),
    (dict(Vt_bits=torch.zeros((33, 2), dtype=torch.int32)), "Vt_bits"),
    (dict(Vt_bits=torch.zeros((32, 3), dtype=torch.int32)), "Vt_bits"),
    (dict(s1=torch.ones(39)), "s1"),
    (dict(s2=torch.ones(71)), "s2"),
])
def test_binary_matmul_rejects_short_buffers(no_library, change, what):
    a = operands()
    a.update(change)
    with pytest.raises(ValueError, match=what):
        nq.binary_matmul(**a)


def test_binary_matmul_vector_output_must_hold_m(no_library):
    a = operands(B=1)
    a["X"] = torch.zeros(70)
    with pytest.raises(ValueError, match="Y"):
        nq.binary_matmul(**a, Y=torch.zeros(39))


@pytest.mark.parametrize("bits, out, what", [
    (torch.zeros((40, 2), dtype=torch.int32), None, "bits"),                      # 70 cols: 3 words
    (torch.zeros((40, 3), dtype=torch.int32), torch.zeros((69, 2), dtype=torch.int32), "out"),
    (torch.zeros((40, 3), dtype=torch.int32), torch.zeros((70, 1), dtype=torch.int32), "out"),
    (torch.zeros((40, 3), dtype=torch.int32), torch.zeros((70, 4), dtype=torch.int32)[:, ::2], "out"),
])
def test_transpose_signs_rejects_short_buffers(no_library, bits, out, what):
    with pytest.raises(ValueError, match=what):
        nq.transpose_signs(bits, 40, 70, out=out)
