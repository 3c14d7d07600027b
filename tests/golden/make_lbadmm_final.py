#!/usr/bin/env python3
"""Write the oracle's end-of-run figures for full-size synthetic layers.

For each workload this runs the CPU oracle (NumPy float64) for the whole
per-layer path on the seeded synthetic layer (synth.make_layer): precondition,
init from the layer's standard-normal draws, the workload's number of ADMM
iterations, balance, scales, signs, and the final errors. It stores the
figures a GPU run is compared with into
``tests/golden/lbadmm_final_<workload>.json``.

It calls only ``oracle/`` (and ``synth/`` for the inputs). Runtime is minutes
for the 4096-wide layers and most of an hour for the 8192 x 28672 layer:

    python tests/golden/make_lbadmm_final.py llama2-7b-attn-4096x4096-r2048
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import lbadmm as O  # noqa: E402
from synth import make_layer  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def run(name: str) -> dict:
    L = make_layer(name)
    wl = L.workload
    t0 = time.perf_counter()
    res = O.lbadmm(L.W, L.d_out, L.d_in, wl.r, rho=wl.rho, iters=wl.iters,
                   svid_steps=wl.svid_steps, EU=L.EU, EV=L.EV)
    dt = time.perf_counter() - t0
    U, V = res.U, res.V
    out = {
        "workload": name,
        "m": wl.m, "n": wl.n, "r": wl.r, "rho": wl.rho,
        "iters": wl.iters, "svid_steps": wl.svid_steps, "seed": wl.seed,
        "rel_err_wtilde": float(res.rel_err_wt),
        "rel_err_w": float(res.rel_err_w),
        "bpw": float(res.bpw),
        "bpw_with_fp16_scales": float(res.bpw_fp16_scales),
        "sigma0": float(res.sigma0),
        # fingerprints of the final balanced latent factors
        "U_fro": float(np.linalg.norm(U)),
        "V_fro": float(np.linalg.norm(V)),
        "U_pos_frac": float(np.mean(U >= 0)),
        "V_pos_frac": float(np.mean(V >= 0)),
        "s1_mean": float(np.mean(res.s1)),
        "s2_mean": float(np.mean(res.s2)),
        "oracle_seconds": dt,
        "source": "oracle.lbadmm.lbadmm (NumPy float64) on synth.make_layer(workload); "
                  "written by tests/golden/make_lbadmm_final.py",
    }
    return out


def main(argv):
    names = argv[1:] or ["llama2-7b-attn-4096x4096-r2048", "llama2-7b-mlp-11008x4096-r1536"]
    for name in names:
        print(f"oracle: {name} ...", flush=True)
        d = run(name)
        path = os.path.join(HERE, f"lbadmm_final_{name}.json")
        with open(path, "w") as f:
            json.dump(d, f, indent=1)
            f.write("\n")
        print(f"wrote {path}: rel_err_wtilde={d['rel_err_wtilde']:.6f} "
              f"({d['oracle_seconds']:.0f} s)", flush=True)


if __name__ == "__main__":
    main(sys.argv)
