"""Plain CPU oracle for applying a low-rank binary layer (test infrastructure).

TEST INFRASTRUCTURE. Only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no
code with the GPU library and never imports it.

Source: [D] "NANOQUANT：大语言模型的高效亚1比特量化 / NanoQuant: Efficient
Sub-1-Bit Quantization of Large Language Models" (paper.rainbus.top),
section 研究动机 (the layer is stored as W ~ diag(s1) U_{+-1} V_{+-1}^T
diag(s2)) and section 技术新颖性 (the authors apply such layers with custom
binary GEMV and GEMM kernels instead of forming W). The pages give no
formula for the product; the plain reading is the matrix product with that
W, taken in the order that never forms W:

    Y = X W^T,  row b:  y_b = s1 * ( S_U ( S_V^T ( s2 * x_b ) ) ),

X being B input vectors of length n (one per row, as activations are laid
out token by token), Y the B outputs of length m. The sign matrices come as
packed bits in the layout of ``oracle.lbadmm.pack_signs`` (bit = [x >= 0],
LSB first, 32 columns per uint32 word).

Everything is float64 NumPy; library matrix products serve as single steps.
"""
from __future__ import annotations

import numpy as np

from .lbadmm import unpack_signs


def binary_matmul(X, U_bits, V_bits, r, s1, s2):
    """Y (B x m) = X W^T for W = diag(s1) S_U S_V^T diag(s2) (m x n).

    X: (B, n); U_bits: (m, ceil(r/32)) uint32; V_bits: (n, ceil(r/32))
    uint32; s1: (m,); s2: (n,). Three products, right to left: scale the
    inputs by s2, project onto the r binary columns of S_V, expand through
    S_U, scale by s1.
    """
    X = np.atleast_2d(np.asarray(X, np.float64))
    SU = unpack_signs(U_bits, r)
    SV = unpack_signs(V_bits, r)
    s1 = np.asarray(s1, np.float64)
    s2 = np.asarray(s2, np.float64)
    Z = X * s2[None, :]          # B x n
    T = Z @ SV                   # B x r: the r binary projections
    return (T @ SU.T) * s1[None, :]   # B x m
