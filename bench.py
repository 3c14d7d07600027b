#!/usr/bin/env python3
"""LB-ADMM throughput on one MI355X.

Workload: a Llama-2-7B attention-projection-shaped layer, W 4096 x 4096 fp32
N(0, 0.02^2) with 1 % of input columns x10, lognormal(0, 0.5)
preconditioners, rank 2048 (1.0 bit per weight), rho = 1, 50 ADMM
iterations, 5 SVID steps (synthetic, seeded; see synth/layers.py).

One step = one whole per-layer run through the C ABI (precondition, init,
50 iterations of U-half + V-half, balance, scales, packing, errors) with the
inputs already resident in HBM. value = ADMM iterations per second over the
timed steps (whole runs, so precondition and finish count against it).

Also reported:
  roofline      the right-hand-side GEMM R = Wt V + rho (Z - Lam), the
                largest kernel: algorithmic 2 m n r flops per launch over its
                average launch duration from HIP events recorded by the
                library on its own stream during the timed steps, against the
                157.3 TFLOP/s fp32 MFMA peak; traffic from the committed
                rocprofv3 counter summary when it matches the current kernel
                source;
  cpu_baseline  the CPU oracle (NumPy float64) on the same layer: a bounded
                number of ADMM iterations on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "llama2-7b-attn-4096x4096-r2048"
FP32_MFMA_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "gemm_rhs_4096x4096_r2048_counters.md")
GEMM_SRC = os.path.join(ROOT, "sub_bit_weight_lb_amd", "csrc", "gemm.hip")


def flops_per_iter(m, n, r):
    """Algorithmic flops of one ADMM iteration (U-half + V-half): two RHS
    GEMMs 4mnr, two Gram products (m+n)r^2 (symmetric count), the triangular
    solves 2(m+n)r^2, two Cholesky factorisations 2 r^3/3."""
    return 4.0 * m * n * r + 3.0 * (m + n) * r * r + 2.0 * r ** 3 / 3.0


def gemm_source_hash():
    return hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()[:16]


def read_traffic(m, n, r, launches_ms):
    """HBM bytes per RHS-GEMM launch from the committed counter summary, or
    None when it is missing or was taken on a different gemm.hip."""
    if not os.path.exists(COUNTER_SUMMARY):
        return None
    txt = open(COUNTER_SUMMARY).read()
    mh = re.search(r"gemm_src_sha256_16:\s*([0-9a-f]{16})", txt)
    mt = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not mh or not mt or mh.group(1) != gemm_source_hash():
        return None
    return float(mt.group(1))


def cpu_baseline(L, budget_s=10.0, max_iters=12, budget_fp32_s=6.0):
    """The CPU oracle on the same layer: a bounded number of ADMM iterations
    in NumPy float64 (the parity oracle; reported as value) and, as a second
    figure, in float32 (the oracle's dtype switch)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import lbadmm as O
    wl = L.workload

    def timed(dtype, budget):
        t0 = time.perf_counter()
        Wt = O.precondition(L.W, L.d_out, L.d_in, dtype)
        st = O.init_state(Wt, wl.r, wl.svid_steps, EU=L.EU, EV=L.EV, dtype=dtype)
        t_prep = time.perf_counter() - t0
        done, t_iter = 0, 0.0
        while done < max_iters and (done == 0 or t_iter * (done + 1) / done < budget):
            t1 = time.perf_counter()
            st = O.iterate(Wt, st, wl.rho, wl.svid_steps, 1, dtype)
            t_iter += time.perf_counter() - t1
            done += 1
        return done, t_iter, t_prep, bool(np.isfinite(st.U).all())

    d64, t64, p64, fin64 = timed(np.float64, budget_s)
    d32, t32, p32, fin32 = timed(np.float32, budget_fp32_s)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": d64 / t64,
        "unit": "iters/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{d64} ADMM iterations (U-half + V-half) of the same {wl.m}x{wl.n} r={wl.r} "
                   f"layer in NumPy float64 after preconditioning and init ({p64:.1f} s, not "
                   f"counted); {t64:.1f} s of iterations"),
        "fp32_value": d32 / t32,
        "fp32_sample": f"{d32} iterations in float32 mode, {t32:.1f} s",
        "host_cpus": len(os.sched_getaffinity(0)),
        "s_per_iter": t64 / d64,
        "finite": fin64 and fin32,
    }


def binary_bench(nq, torch, dev, reps=20, replays=5):
    """nq_binary_matmul (Y = X W^T for W = diag(s1) S_U S_V^T diag(s2)) on the
    factorised-layer shapes. Random sign words on the device. Calls are
    captured in a HIP graph (no host overhead in the timing) and replayed;
    "warm" reuses one set of bits, "cold" rotates through copies of the bits
    totalling > 256 MB (more than the last-level cache), so each call reads
    its bits from HBM. Algorithmic bytes per call: the bits, X, Y, s1, s2 and
    the B r projections written and read back."""
    out = []
    g = torch.Generator(device="cpu").manual_seed(0)
    for (m, n, r) in ((4096, 4096, 2048), (11008, 4096, 1536), (8192, 28672, 6144)):
        wu, wv = (r + 31) // 32, (n + 31) // 32
        bits_bytes = 4 * (m * wu + r * wv)
        ncopy = max(1, -(-320 * 2**20 // bits_bytes))
        U = [torch.randint(-2**31, 2**31 - 1, (m, wu), dtype=torch.int32, generator=g).to(dev)
             for _ in range(ncopy)]
        Vt = [torch.randint(-2**31, 2**31 - 1, (r, wv), dtype=torch.int32, generator=g).to(dev)
              for _ in range(ncopy)]
        s1 = torch.rand(m, generator=g).to(dev)
        s2 = torch.rand(n, generator=g).to(dev)
        for B in (1, 8, 16):
            X = torch.randn(B, n, generator=g).to(dev)
            Y = torch.empty(B, m, device=dev)
            work = torch.empty(8 * B * r, device=dev)
            nq.binary_matmul(U[0], Vt[0], s1, s2, X, r, Y=Y, work=work)
            ref = Y.clone()
            res = {"m": m, "n": n, "r": r, "B": B}
            alg = bits_bytes + 4 * (B * n + B * m + m + n + 2 * B * r)
            for mode, sets in (("warm", [0] * reps), ("cold", [i % ncopy for i in range(reps)])):
                st = torch.cuda.Stream()
                st.wait_stream(torch.cuda.current_stream())
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.stream(st):
                    nq.binary_matmul(U[0], Vt[0], s1, s2, X, r, Y=Y, work=work)  # warm-up on st
                    torch.cuda.synchronize()
                    with torch.cuda.graph(graph, stream=st):
                        for i in sets:
                            nq.binary_matmul(U[i], Vt[i], s1, s2, X, r, Y=Y, work=work)
                torch.cuda.synchronize()
                graph.replay()
                torch.cuda.synchronize()
                if mode == "warm" and not torch.equal(Y, ref):
                    raise RuntimeError("graph replay differs from the eager call")
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(replays):
                    graph.replay()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / (replays * reps)
                res[f"{mode}_us"] = round(us, 2)
                res[f"{mode}_GBps"] = round(alg / us / 1e3, 1)
                del graph
            res["alg_bytes"] = alg
            res["cold_frac_of_8TBps"] = round(res["cold_GBps"] / 8000.0, 4)
            print(json.dumps(res), flush=True)
            out.append(res)
        del U, Vt
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single-stream", action="store_true")
    ap.add_argument("--iters", type=int, default=None, help="override ADMM iterations per run")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (counter calibration)")
    ap.add_argument("--kernels", action="store_true",
                    help="only run the GEMM kernels alone on the layer's shapes, 20 launches "
                         "each (for a kernel-trace profile of their standalone durations)")
    ap.add_argument("--binary", action="store_true",
                    help="only time the binary-layer product (nq_binary_matmul) on the layer "
                         "shapes, warm and with its sign bits rotated through > 256 MB")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the per-layer path runs on a single GPU)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        # A plain copy of known size: 256 MiB read + 256 MiB written per launch.
        n = 64 * 1024 * 1024
        src = torch.rand(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": 4 * n, "bytes_written": 4 * n,
                          "launches": 4}), flush=True)
        return

    import sub_bit_weight_lb_amd as nq
    from synth import make_layer

    dev = torch.device("cuda:0")
    if args.kernels:
        # RHS shape (m x n times n x r), solve shape (m x r times r x r), Gram
        # (n x r); op_gemm_rhs also runs a transpose kernel per call, which a
        # kernel trace lists on its own line
        g = torch.Generator(device="cpu").manual_seed(0)
        from synth.layers import WORKLOADS
        wl = WORKLOADS[WORKLOAD]
        for (mm, kk, nn) in ((wl.m, wl.n, wl.r), (wl.m, wl.r, wl.r)):
            a = torch.randn(mm, kk, generator=g).to(dev)
            b = torch.randn(kk, nn, generator=g).to(dev)
            for _ in range(20):
                nq.op_gemm_rhs(a, b)
            torch.cuda.synchronize()
            print(f"gemm {mm}x{nn}x{kk}: 20 launches", flush=True)
        v = (0.05 * torch.randn(wl.n, wl.r, generator=g)).to(dev)
        for _ in range(20):
            nq.op_gram(v, rho=wl.rho)
        torch.cuda.synchronize()
        print(f"gram {wl.n}x{wl.r}: 20 launches", flush=True)
        return
    if args.binary:
        print(json.dumps({"binary_matmul": binary_bench(nq, torch, dev)}), flush=True)
        return
    L = make_layer(WORKLOAD)
    wl = L.workload
    m, n, r = wl.m, wl.n, wl.r
    iters = wl.iters if args.iters is None else args.iters

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    W, d_out, d_in, EU, EV = t(L.W), t(L.d_out), t(L.d_in), t(L.EU), t(L.EV)
    print(f"bench: {WORKLOAD} iters={iters} warmup={args.warmup} steps={args.steps}",
          file=sys.stderr, flush=True)
    # Phase breakdown: one untimed run on a handle that times every phase
    # (each event pair costs a little device time, ~1.5 % over a run).
    hp = nq.LBADMM(m, n, r, rho=wl.rho, iters=iters, svid_steps=wl.svid_steps,
                   compute_error=True, single_stream=args.single_stream, profile=True)
    out = hp.alloc_outputs(dev)
    hp.run(W, d_out, d_in, EU, EV, out=out, want_stats=False)
    phases = hp.profile(reset=True)
    hp.close()
    # Timed runs: HIP events around the RHS GEMM only, on its own stream
    # (the roofline's launch duration); no other events in the timed region.
    h = nq.LBADMM(m, n, r, rho=wl.rho, iters=iters, svid_steps=wl.svid_steps,
                  compute_error=True, single_stream=args.single_stream, profile="rhs")
    for _ in range(args.warmup):
        h.run(W, d_out, d_in, EU, EV, out=out, want_stats=False)
    torch.cuda.synchronize()
    h.profile(reset=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        h.run(W, d_out, d_in, EU, EV, out=out, want_stats=False)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = h.profile(reset=True)
    status, stats = nq.lbadmm_query(h.handle)
    if status != 0:
        raise SystemExit(f"run reported {nq.status_string(status)}")
    h.close()

    elapsed = t1 - t0
    ms_per_step = 1e3 * elapsed / args.steps
    value = args.steps * iters / elapsed
    F = flops_per_iter(m, n, r)
    rhs_ms, rhs_n = prof["gemm_rhs"]
    rhs_avg_s = rhs_ms / max(rhs_n, 1) / 1e3
    rhs_flops = 2.0 * m * n * r
    achieved = rhs_flops / rhs_avg_s / 1e12
    traffic = read_traffic(m, n, r, rhs_avg_s)
    line = {
        "metric": "LB-ADMM iters/s on 4096x4096 r=2048 fp32 layer; % of fp32 MFMA peak",
        "value": round(value, 3),
        "unit": "iters/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "m": m, "n": n, "r": r, "rho": wl.rho,
                   "admm_iters_per_step": iters, "svid_steps": wl.svid_steps,
                   "parallelism": "single-gpu"},
        "fp32_mfma_peak_frac": round(value * F / (FP32_MFMA_PEAK_TFLOPS * 1e12), 4),
        "factorised_weights_per_s": round(args.steps * m * n / elapsed, 1),
        "flops_per_iter": F,
        "roofline": {
            "kernel": "gemm_nt_kernel<kEpiRhs> (R = Wt V + rho (Z - Lam), V read as V^T)",
            "note": ("timed as it runs in the pipeline: on 7 of the 8 XCDs (the eighth runs the "
                     "Cholesky chain's diagonal work) and yielding issue cycles to the chain "
                     "(s_sleep after each K step); the same kernel alone on the whole chip: "
                     "see the standalone kernel profile"),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": FP32_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / FP32_MFMA_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(rhs_avg_s * 1e3, 4),
            "launches": rhs_n,
            "flops_per_launch": rhs_flops,
        },
        # from one untimed run with every phase timed (the chain phase is the
        # Gram plus the Cholesky chain; phases of different streams overlap)
        "phase_ms_per_iter": {p: round(phases[p][0] / max(iters, 1), 4)
                              for p in ("gemm_rhs", "gemm_solve", "chain", "svid")},
        "phase_ms_per_step": {p: round(phases[p][0], 3) for p in ("prep", "finish")},
        "phase_source": "one untimed run with every phase timed",
        # the solve GEMM runs alone on the chip, on the critical path
        "solve_gemm": {
            "flops_per_launch": 2.0 * m * r * r,
            "avg_launch_ms": round(phases["gemm_solve"][0] / max(phases["gemm_solve"][1], 1), 4),
            "tflops": round(2.0 * m * r * r / (phases["gemm_solve"][0] / max(phases["gemm_solve"][1], 1)
                                                / 1e3) / 1e12, 2),
            "frac_of_peak": round(2.0 * m * r * r / (phases["gemm_solve"][0]
                                                      / max(phases["gemm_solve"][1], 1) / 1e3)
                                  / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
            "source": "the untimed run with every phase timed",
        },
        "rel_err_wtilde": stats["rel_err_wtilde"],
        "rel_err_w": stats["rel_err_w"],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(L)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
