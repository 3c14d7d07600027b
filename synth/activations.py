"""Seeded synthetic activation samples for the calibration statistics.

Stand-in for the pages' calibration pass (128 WikiText-2 samples of 2048
tokens run through the model; no dataset or weights are used here): a token
x feature matrix whose features have lognormal(0, 1) scales, nonzero means
(0.3 standard deviations, drawn per feature) and a fraction of outlier
features scaled x20, the heavy-tailed channel structure of LLM activations.
Random numbers only: none of the method's arithmetic.
"""
from __future__ import annotations

import numpy as np

# 128 samples x 2048 tokens, the pages' calibration set
CALIB_TOKENS = 128 * 2048


def feature_profile(p: int, seed: int, outlier_frac: float = 0.01):
    """(scale, mean) per feature, float64, and the generator to draw tokens
    with afterwards."""
    rng = np.random.default_rng(seed)
    scale = rng.lognormal(0.0, 1.0, p)
    k = int(round(outlier_frac * p))
    if k:
        scale[rng.choice(p, k, replace=False)] *= 20.0
    mean = 0.3 * rng.standard_normal(p) * scale
    return scale, mean, rng


def make_activations(N: int, p: int, seed: int, outlier_frac: float = 0.01,
                     dtype=np.float32) -> np.ndarray:
    """N tokens x p features."""
    scale, mean, rng = feature_profile(p, seed, outlier_frac)
    Z = rng.standard_normal((N, p), dtype=np.float32)
    Z *= scale.astype(np.float32)
    Z += mean.astype(np.float32)
    return Z.astype(dtype, copy=False)
