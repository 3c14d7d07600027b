"""Seeded synthetic layers shaped like the pages' Llama-2 workloads.

NanoQuant (arXiv 2602.06694) measures on Llama-2-7B / Llama-2-70B linear
layers (digest page paper.rainbus.top, sections "实验结果" and the
structured-data table). No model weights are available here, so every layer
is drawn from a seeded PCG64 generator with the shapes of those layers and
the value distributions listed in ``WORKLOADS``.

Draw order for one layer (all draws in float64, then cast to float32):
    W (m x n), outlier input-column indices, d_in (n), d_out (m),
    EU (m x r, standard normal), EV (n x r, standard normal).

EU and EV are the random numbers the initialisation consumes; the scale
applied to them is method arithmetic and lives on each side separately.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    m: int                      # output features (rows of W)
    n: int                      # input features (columns of W)
    r: int                      # rank of the binary factors
    rho: float                  # ADMM penalty
    iters: int                  # ADMM iterations (each: U-half then V-half)
    svid_steps: int             # power/ALS steps inside SVID
    seed: int
    dist: str = "normal"        # "normal" or "t4" (Student-t, nu = 4)
    std: float = 0.02           # target standard deviation of W entries
    outlier_frac: float = 0.0   # fraction of input columns scaled up
    outlier_scale: float = 1.0
    d_sigma: float = 0.5        # lognormal(0, d_sigma) preconditioner entries

    @property
    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.n))


@dataclass
class LayerInputs:
    workload: Workload
    W: np.ndarray        # float32 (m, n), row-major [out, in]
    d_out: np.ndarray    # float32 (m,)
    d_in: np.ndarray     # float32 (n,)
    EU: np.ndarray       # float32 (m, r) standard-normal draws
    EV: np.ndarray       # float32 (n, r) standard-normal draws
    outlier_cols: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))


def _block(seed0: int) -> List[Workload]:
    names = ["q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj"]
    shapes = [(4096, 4096)] * 4 + [(11008, 4096), (11008, 4096), (4096, 11008)]
    ranks = [2048] * 4 + [2970] * 3
    return [Workload(f"llama2-7b-block.{nm}", m, n, r, 1.0, 40, 5, seed0 + i)
            for i, (nm, (m, n), r) in enumerate(zip(names, shapes, ranks))]


WORKLOADS: Dict[str, Workload] = {
    # 256 x 512, r = 128 (0.75 bit/weight): small enough for the fp64 oracle in seconds.
    "tiny-256x512-r128": Workload("tiny-256x512-r128", 256, 512, 128, 1.0, 20, 5, 1),
    # Llama-2-7B attention projection, 1 % outlier input channels x10, r = 2048 (1.0 bit/weight).
    "llama2-7b-attn-4096x4096-r2048": Workload(
        "llama2-7b-attn-4096x4096-r2048", 4096, 4096, 2048, 1.0, 50, 5, 2,
        outlier_frac=0.01, outlier_scale=10.0),
    # Llama-2-7B MLP gate/up projection, heavy-tailed entries, r = 1536 (~0.52 bit/weight).
    "llama2-7b-mlp-11008x4096-r1536": Workload(
        "llama2-7b-mlp-11008x4096-r1536", 11008, 4096, 1536, 0.5, 50, 5, 3,
        dist="t4", d_sigma=0.7),
    # Llama-2-70B MLP down projection, 0.5 % outlier input channels x8, r = 6144.
    "llama2-70b-down-8192x28672-r6144": Workload(
        "llama2-70b-down-8192x28672-r6144", 8192, 28672, 6144, 1.0, 30, 5, 5,
        std=0.015, outlier_frac=0.005, outlier_scale=8.0),
}
for _w in _block(40):
    WORKLOADS[_w.name] = _w

BLOCK_LAYERS: List[str] = [w.name for w in _block(40)]


def make_layer(workload, seed: Optional[int] = None, with_init: bool = True) -> LayerInputs:
    """Draw one synthetic layer. ``workload`` is a Workload or a WORKLOADS key."""
    wl = WORKLOADS[workload] if isinstance(workload, str) else workload
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    m, n, r = wl.m, wl.n, wl.r
    if wl.dist == "normal":
        W = rng.standard_normal((m, n)) * wl.std
    elif wl.dist == "t4":
        # Student-t with nu = 4 has variance nu / (nu - 2) = 2.
        W = rng.standard_t(4.0, size=(m, n)) * (wl.std / np.sqrt(2.0))
    else:
        raise ValueError(f"unknown distribution {wl.dist!r}")
    cols = np.zeros(0, np.int64)
    if wl.n_outliers > 0:
        cols = np.sort(rng.choice(n, size=wl.n_outliers, replace=False))
        W[:, cols] *= wl.outlier_scale
    d_in = rng.lognormal(0.0, wl.d_sigma, size=n)
    d_out = rng.lognormal(0.0, wl.d_sigma, size=m)
    W32 = W.astype(np.float32)
    del W
    if with_init:
        EU = rng.standard_normal((m, r)).astype(np.float32)
        EV = rng.standard_normal((n, r)).astype(np.float32)
    else:
        EU = np.zeros((0, r), np.float32)
        EV = np.zeros((0, r), np.float32)
    return LayerInputs(wl, W32, d_out.astype(np.float32), d_in.astype(np.float32),
                       EU, EV, cols)


def make_tiny(m: int, n: int, r: int, seed: int, rho: float = 1.0, iters: int = 3,
              svid_steps: int = 5, dist: str = "normal", std: float = 0.02,
              d_sigma: float = 0.5, outlier_frac: float = 0.0,
              outlier_scale: float = 1.0) -> LayerInputs:
    """An ad-hoc layer of any shape (for parity cases: ragged, tiny, degenerate)."""
    wl = Workload(f"adhoc-{m}x{n}-r{r}-s{seed}", m, n, r, rho, iters, svid_steps, seed,
                  dist=dist, std=std, outlier_frac=outlier_frac,
                  outlier_scale=outlier_scale, d_sigma=d_sigma)
    return make_layer(wl)


def with_iters(workload: Workload, iters: int) -> Workload:
    return replace(workload, iters=iters)
