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

--workload NAME times another synthetic layer of synth/layers.py instead
(the tiny 256 x 512 layer, the 11008 x 4096 r = 1536 MLP layer, the
8192 x 28672 r = 6144 layer), or 'llama2-7b-block': the seven layers of one
Llama-2-7B-shaped block run one after the other in each step, value = all
their iterations per second.

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
BLOCK = "llama2-7b-block"
METRIC = "LB-ADMM iters/s on 4096x4096 r=2048 fp32 layer; % of fp32 MFMA peak"
FP32_MFMA_PEAK_TFLOPS = 157.3
BF16_MFMA_PEAK_TFLOPS = 2500.0
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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bpw(m, n, r, scale_bits=16):
    """Bits per weight of the factorised layer: the sign bits r (m + n), plus
    the two scale vectors at `scale_bits` each (fp16 by default)."""
    return (r * (m + n) + scale_bits * (m + n)) / (m * n)


def hbm_bench(nq, torch, dev, L, reps=20):
    """The HBM-bound kernels alone at the layer's shape, with HIP events: the
    SVID + dual update (one launch per update, on the state a run leaves) for
    each factor, and whole runs of one iteration split by phase (prep =
    precondition + init, finish = balance + scales + packing + error)."""
    wl = L.workload
    m, n, r = wl.m, wl.n, wl.r

    def t(x):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    W, d_out, d_in, EU, EV = t(L.W), t(L.d_out), t(L.d_in), t(L.EU), t(L.EV)
    h = nq.LBADMM(m, n, r, rho=wl.rho, iters=1, svid_steps=wl.svid_steps, compute_error=True,
                  init_draws=True,
                  profile=True)
    out = h.alloc_outputs(dev)
    h.run(W, d_out, d_in, EU, EV, out=out, want_stats=False)
    h.profile(reset=True)
    for _ in range(reps):
        h.run(W, d_out, d_in, EU, EV, out=out, want_stats=False)
    ph = h.profile(reset=True)
    res = {"prep_ms": round(ph["prep"][0] / ph["prep"][1], 4),
           "finish_ms": round(ph["finish"][0] / ph["finish"][1], 4)}
    for f, rows in ((0, m), (1, n)):
        ms = h.time_svid(f, reps=reps)
        gbs = 16.0 * rows * r / (ms * 1e-3) / 1e9
        res["svid_" + "UV"[f]] = {"avg_us": round(ms * 1e3, 2), "bytes": 16 * rows * r,
                                  "GBps": round(gbs, 1), "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4)}
    h.close()
    return res


def cpu_baseline(layers, budget_s=10.0, budget_fp32_s=6.0, max_halves=24):
    """The CPU oracle on the same workload: ADMM half-iterations (oracle
    admm_half, U then V, as oracle iterate runs them) in NumPy float64 (the
    parity oracle; reported as value) and, as a second figure, in float32
    (the oracle's dtype switch). Each distinct layer shape of the workload is
    sampled for its share of the budget (at least one half-iteration); the
    workload's iterations/s is the total of its iterations over the time the
    sampled rates give for all its layers."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import lbadmm as O

    shapes = {}
    for L in layers:
        wl = L.workload
        shapes.setdefault((wl.m, wl.n, wl.r), L)

    def timed(L, dtype, budget):
        wl = L.workload
        t0 = time.perf_counter()
        Wt = O.precondition(L.W, L.d_out, L.d_in, dtype)
        st = O.init_state(Wt, wl.r, wl.svid_steps, EU=L.EU, EV=L.EV, dtype=dtype)
        t_prep = time.perf_counter() - t0
        halves, t_run = 0, 0.0
        while halves < max_halves and (halves == 0 or t_run * (halves + 1) / halves < budget):
            t1 = time.perf_counter()
            if halves % 2 == 0:
                st.U, st.Z_U, st.Lam_U, _, _ = O.admm_half(Wt, st.V, st.Z_U, st.Lam_U, wl.rho,
                                                           wl.svid_steps)
            else:
                st.V, st.Z_V, st.Lam_V, _, _ = O.admm_half(Wt.T, st.U, st.Z_V, st.Lam_V, wl.rho,
                                                           wl.svid_steps)
            t_run += time.perf_counter() - t1
            halves += 1
        fin = bool(np.isfinite(st.U).all() and np.isfinite(st.V).all())
        del Wt, st
        return halves, t_run, t_prep, fin

    res = {}
    for dt, budget in ((np.float64, budget_s), (np.float32, budget_fp32_s)):
        rates, notes, fin = {}, [], True
        for key, L in shapes.items():
            h, t, tp, f = timed(L, dt, budget / len(shapes))
            print(f"cpu baseline: {np.dtype(dt).name} {key}: {h} half-iterations in {t:.1f} s",
                  file=sys.stderr, flush=True)
            rates[key] = 2.0 * t / h                         # seconds per iteration
            fin = fin and f
            notes.append(f"{h} half-iterations of {key[0]}x{key[1]} r={key[2]} "
                         f"({t:.1f} s; preconditioning and init {tp:.1f} s, not counted)")
        iters = sum(L.workload.iters for L in layers)
        secs = sum(L.workload.iters * rates[(L.workload.m, L.workload.n, L.workload.r)]
                   for L in layers)
        res[dt] = (iters / secs, "; ".join(notes), fin, secs / iters)
    pools = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in pools] + [1])
    blas = sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
                   for i in pools if i.get("user_api") == "blas"})
    v64, s64, f64, spi = res[np.float64]
    v32, s32, f32, _ = res[np.float32]
    return {
        "value": v64,
        "unit": "iters/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"NumPy float64: {s64}",
        "fp32_value": v32,
        "fp32_sample": f"float32 mode: {s32}",
        "host_cpus": len(os.sched_getaffinity(0)),
        "blas": ", ".join(blas) or "unknown",
        "cpu_model": cpu_model(),
        "s_per_iter": spi,
        "finite": f64 and f32,
    }


def lw_bench(nq, torch, dev, p=4096, chunk=16384, reps=3):
    """The Ledoit-Wolf preconditioner of one layer side: the pages'
    calibration set (128 x 2048 tokens) of p-feature activations, resident in
    HBM as chunk-row pieces (seeded on the device with the feature profile of
    synth.activations), accumulated chunk by chunk and finalised. Algorithmic
    work: the second moment's Gram, N p^2 flops (symmetric count); HBM bytes:
    the samples read twice (staging and row norms), 8 N p."""
    import numpy as np
    from synth.activations import CALIB_TOKENS, feature_profile
    N = CALIB_TOKENS
    scale, mean, _ = feature_profile(p, 0)
    sc = torch.from_numpy(scale.astype(np.float32)).to(dev)
    mu = torch.from_numpy(mean.astype(np.float32)).to(dev)
    g = torch.Generator(device=dev).manual_seed(0)
    chunks = [torch.randn(chunk, p, generator=g, device=dev) * sc + mu for _ in range(N // chunk)]
    torch.cuda.synchronize()
    lw = nq.LedoitWolf(p, chunk)
    res = {"p": p, "tokens": N, "chunk_rows": chunk}
    times = []
    for rep in range(reps + 1):
        lw.reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for c in chunks:
            lw.accumulate(c)
        d, s = lw.finalize()
        e1.record()
        torch.cuda.synchronize()
        if rep:
            times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    flops = float(N) * p * p
    res.update({"ms": round(ms, 3), "tokens_per_s": round(N / (ms * 1e-3), 1),
                "gram_flops": flops, "whole_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                "whole_frac_of_fp32_peak": round(flops / (ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
                "shrinkage": s, "d_min": float(d.min()), "d_max": float(d.max())})
    lw.close()
    return res


def lw_cpu_baseline(p=4096, tokens=128):
    """The oracle (oracle/precond.py) on a bounded sample of the same
    workload: `tokens` tokens of p features; tokens/s."""
    from oracle import precond as P
    from synth.activations import make_activations
    Z = make_activations(tokens, p, 0)
    t0 = time.perf_counter()
    P.diag_preconditioner(Z)
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "kind": "oracle",
            "sample": f"{tokens} tokens x {p} features, NumPy float64, {dt:.1f} s"}


def ste_bench(nq, torch, dev, samples=128, seq=2048, batch=4, epochs=8, admm_iters=50):
    """STE refinement of the 4096 x 4096, r = 2048 layer with the pages'
    settings: the calibration set (128 samples x 2048 tokens) of activations
    seeded on the device (feature profile of synth.activations), targets
    Y = X W^T, 8 epochs of shuffled batches of 4 samples (8192 tokens), lr
    1e-4 -> 1e-6 on the cosine schedule, from the factors of an LB-ADMM run.
    Algorithmic work per step: six products, 6 T r (m + n) flops. Four have
    a +-1 factor and run on the bf16 matrix cores with the other factor as
    three exact bf16 terms (3x the flops there), two on the fp32 ones; the
    step's roofline is the time both sets would take at their peaks."""
    import numpy as np
    from synth import make_layer
    from synth.activations import feature_profile
    L = make_layer(WORKLOAD)
    wl = L.workload
    m, n, r = wl.m, wl.n, wl.r

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    W = t(L.W)
    with nq.LBADMM(m, n, r, rho=wl.rho, iters=admm_iters, svid_steps=wl.svid_steps,
                   init_draws=True) as h:
        res = h.run(W, t(L.d_out), t(L.d_in), t(L.EU), t(L.EV))
    N = samples * seq
    scale, mean, _ = feature_profile(n, 0)
    sc = torch.from_numpy(scale.astype(np.float32)).to(dev)
    mu = torch.from_numpy(mean.astype(np.float32)).to(dev)
    g = torch.Generator(device=dev).manual_seed(0)
    X = torch.randn(N, n, generator=g, device=dev) * sc + mu
    Y = X @ W.T
    rng = np.random.default_rng(0)
    batches = []
    for _ in range(epochs):
        order = rng.permutation(samples)
        for b in range(0, samples, batch):
            idx = (order[b:b + batch, None] * seq + np.arange(seq)[None, :]).reshape(-1)
            batches.append(torch.from_numpy(idx.astype(np.int32)).to(dev))
    T = batch * seq
    out = {"m": m, "n": n, "r": r, "tokens_per_step": T, "steps": len(batches),
           "epochs": epochs, "schedule": "cosine 1e-4 -> 1e-6, Adam"}
    with nq.STERefiner(m, n, r, T) as ste:
        # untimed: the loss of every step (each read waits for the GPU)
        ste.set_params(res.U, res.V, res.s1, res.s2)
        losses = ste.refine(X, Y, batches)
        out["loss_first"] = losses[0]
        out["loss_last"] = losses[-1]
        out["loss_epoch_means"] = [round(float(np.mean(losses[e * len(batches) // epochs:
                                                            (e + 1) * len(batches) // epochs])), 6)
                                   for e in range(epochs)]
        # timed: the same schedule from the same start, no reads
        ste.set_params(res.U, res.V, res.s1, res.s2)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ste.refine(X, Y, batches, losses=False, check_rows=False)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
    flops = 6.0 * T * r * (m + n)
    sign_flops = 4.0 * T * r * (m + n)          # P, Q, dP, dA
    fp32_flops = flops - sign_flops             # dU, dV
    # the step at both peaks: 3 bf16 products per sign product
    t_roof = 3.0 * sign_flops / (BF16_MFMA_PEAK_TFLOPS * 1e12) + fp32_flops / (FP32_MFMA_PEAK_TFLOPS * 1e12)
    step_ms = ms / len(batches)
    out.update({"ms_total": round(ms, 2), "ms_per_step": round(step_ms, 3),
                "steps_per_s": round(1e3 / step_ms, 2), "tokens_per_s": round(T * 1e3 / step_ms, 1),
                "flops_per_step": flops, "tflops": round(flops / (step_ms * 1e-3) / 1e12, 2),
                "roofline_ms_per_step": round(t_roof * 1e3, 3),
                "frac_of_roofline": round(t_roof * 1e3 / step_ms, 4)})
    return out


def ste_cpu_baseline(tokens=2048):
    """The oracle (oracle/ste.py) on a bounded sample of the same workload:
    one step (gradients + Adam) on `tokens` tokens of the 4096 x 4096,
    r = 2048 layer from a random start, scaled to 8192-token steps."""
    import numpy as np
    from oracle import ste as S
    from synth.activations import make_activations
    rng = np.random.default_rng(0)
    m = n = 4096
    r = 2048
    W = 0.02 * rng.standard_normal((m, n))
    X = make_activations(tokens, n, 0).astype(np.float64)
    Y = X @ W.T
    U, V = rng.standard_normal((m, r)), rng.standard_normal((n, r))
    s1, s2 = np.full(m, 0.02), np.full(n, 0.02)
    t0 = time.perf_counter()
    st = S.adam_init([U, V, s1, s2])
    S.adam_step([U, V, s1, s2], S.grads(X, Y, U, V, s1, s2), st, 1e-4)
    dt = time.perf_counter() - t0
    return {"value": 1.0 / (dt * 8192 / tokens), "unit": "steps/s (8192-token steps)",
            "kind": "oracle", "sample": f"one step on {tokens} tokens, NumPy float64, {dt:.1f} s"}


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
            work = torch.empty(nq.binary_matmul_work_floats(B, n, r), device=dev)
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
    ap.add_argument("--hbm", action="store_true",
                    help="only time the HBM-bound kernels (SVID + dual update, prep, finish) "
                         "on the layer's shape (for counter and kernel-trace profiles)")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="a synthetic layer (synth.layers.WORKLOADS) or 'llama2-7b-block' "
                         "(the seven layers of one Llama-2-7B-shaped block, run one after the "
                         "other in each step)")
    ap.add_argument("--solver", default=None,
                    help="METHOD:STEPS, an iterative solve of each half's system instead of the "
                         "Cholesky factor: cg (conjugate gradients) or gd (steepest descent), "
                         "STEPS steps per half, e.g. cg:8")
    ap.add_argument("--ste", action="store_true",
                    help="only time the STE refinement (nq_ste_*) of the 4096 x 4096, r = 2048 "
                         "layer: 8 epochs of 4-sample batches over 128 x 2048 tokens")
    ap.add_argument("--lw", action="store_true",
                    help="only time the Ledoit-Wolf diagonal preconditioner (nq_lw_*) on the "
                         "calibration set's 128 x 2048 tokens of 4096 features")
    ap.add_argument("--binary", action="store_true",
                    help="only time the binary-layer product (nq_binary_matmul) on the layer "
                         "shapes, warm and with its sign bits rotated through > 256 MB")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the per-layer path runs on a single GPU)", file=sys.stderr)
        sys.exit(2)

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
        wl = WORKLOADS[workload_layers(args.workload)[0]]
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
    if args.ste:
        out = {"ste_refinement": ste_bench(nq, torch, dev)}
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = ste_cpu_baseline()
        print(json.dumps(out), flush=True)
        return
    if args.lw:
        out = {"ledoit_wolf": lw_bench(nq, torch, dev)}
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = lw_cpu_baseline()
        print(json.dumps(out), flush=True)
        return
    names = workload_layers(args.workload)
    if args.hbm:
        print(json.dumps({"hbm_kernels": hbm_bench(nq, torch, dev, make_layer(names[0]))}),
              flush=True)
        return
    layers = [make_layer(nm) for nm in names]
    solver = None
    if args.solver:
        meth, _, k = args.solver.partition(":")
        solver = (meth, int(k))
    line = measure(nq, torch, dev, args, layers, solver)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(layers)
    print(json.dumps(line), flush=True)


def workload_layers(name):
    """The layer names of a workload: one synthetic layer, or the seven
    layers of the Llama-2-7B-shaped block."""
    from synth.layers import BLOCK_LAYERS, WORKLOADS
    if name == BLOCK:
        return list(BLOCK_LAYERS)
    if name not in WORKLOADS:
        raise SystemExit(f"unknown workload {name!r}; one of {sorted(WORKLOADS) + [BLOCK]}")
    return [name]


def measure(nq, torch, dev, args, layers, solver=None):
    """One step = one whole per-layer run of every layer of the workload
    through the C ABI, inputs resident in HBM."""
    import numpy as np

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    runs = []
    for L in layers:
        wl = L.workload
        iters = wl.iters if args.iters is None else args.iters
        ins = [t(x) for x in (L.W, L.d_out, L.d_in, L.EU, L.EV)]
        runs.append((wl, iters, ins))
    name = args.workload
    print(f"bench: {name} ({len(layers)} layer(s)) warmup={args.warmup} steps={args.steps}",
          file=sys.stderr, flush=True)
    # Phase breakdown: one untimed run per layer on a handle that times every
    # phase (each event pair costs a little device time, ~1.5 % over a run).
    phases_all = []
    for wl, iters, ins in runs:
        hp = nq.LBADMM(wl.m, wl.n, wl.r, rho=wl.rho, iters=iters, svid_steps=wl.svid_steps,
                       compute_error=True, single_stream=args.single_stream, profile=True,
                       init_draws=True,
                       solver=solver)
        out = hp.alloc_outputs(dev)
        hp.run(*ins, out=out, want_stats=False)
        phases_all.append(hp.profile(reset=True))
        hp.close()
        del out
    # Timed runs: HIP events around the RHS GEMM only, on its own stream (the
    # roofline's launch duration); no other events in the timed region.
    handles = []
    for wl, iters, ins in runs:
        h = nq.LBADMM(wl.m, wl.n, wl.r, rho=wl.rho, iters=iters, svid_steps=wl.svid_steps,
                      compute_error=True, single_stream=args.single_stream, profile="rhs",
                      init_draws=True,
                      solver=solver)
        handles.append((h, h.alloc_outputs(dev)))

    def step():
        for (h, out), (_, _, ins) in zip(handles, runs):
            h.run(*ins, out=out, want_stats=False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for h, _ in handles:
        h.profile(reset=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rhs_ms, rhs_n, rhs_flops, stats_all, svid = 0.0, 0, 0.0, [], {}
    for (h, _), (wl, iters, _) in zip(handles, runs):
        prof = h.profile(reset=True)
        status, stats = nq.lbadmm_query(h.handle)
        if status != 0:
            raise SystemExit(f"{wl.name}: run reported {nq.status_string(status)}")
        stats_all.append(stats)
        ms, cnt = prof["gemm_rhs"]
        rhs_ms += ms
        rhs_n += cnt
        rhs_flops += cnt * 2.0 * wl.m * wl.n * wl.r
        # The SVID + dual update alone (one persistent launch per update), on
        # the state the last run left: algorithmic bytes 16 per element of
        # the factor (read the latent and Lam, write Lam and P).
        key = f"{wl.m}x{wl.n}-r{wl.r}"
        if key not in svid:
            svid[key] = {}
            for f, rows in ((0, wl.m), (1, wl.n)):
                ms = h.time_svid(f, reps=20)
                gbs = 16.0 * rows * wl.r / (ms * 1e-3) / 1e9
                svid[key]["UV"[f]] = {"avg_us": round(ms * 1e3, 2), "bytes": 16 * rows * wl.r,
                                      "GBps": round(gbs, 1),
                                      "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4)}
        h.close()

    elapsed = t1 - t0
    iters_step = sum(iters for _, iters, _ in runs)
    value = args.steps * iters_step / elapsed
    F = sum(iters * flops_per_iter(wl.m, wl.n, wl.r) for wl, iters, _ in runs)
    rhs_avg_s = rhs_ms / max(rhs_n, 1) / 1e3
    achieved = rhs_flops / max(rhs_n, 1) / rhs_avg_s / 1e12
    single = len(runs) == 1
    wl0 = runs[0][0]
    traffic = (read_traffic(wl0.m, wl0.n, wl0.r, rhs_avg_s)
               if single and name == WORKLOAD else None)
    weights = sum(wl.m * wl.n for wl, _, _ in runs)
    bits = sum(wl.r * (wl.m + wl.n) for wl, _, _ in runs)
    scale_bits = sum(16 * (wl.m + wl.n) for wl, _, _ in runs)
    cfg = {"workload": name, "layers": len(runs), "parallelism": "single-gpu",
           "solve": "cholesky" if solver is None else f"{solver[0]} x{solver[1]}"}
    if single:
        cfg.update({"m": wl0.m, "n": wl0.n, "r": wl0.r, "rho": wl0.rho,
                    "admm_iters_per_step": runs[0][1], "svid_steps": wl0.svid_steps})
    else:
        cfg["shapes"] = [f"{wl.m}x{wl.n}-r{wl.r}" for wl, _, _ in runs]
        cfg["admm_iters_per_step"] = iters_step
    line = {
        "metric": (METRIC if name == WORKLOAD
                   else f"LB-ADMM iters/s on {name} fp32; % of fp32 MFMA peak"),
        "value": round(value, 3),
        "unit": "iters/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": cfg,
        "fp32_mfma_peak_frac": round(args.steps * F / elapsed / (FP32_MFMA_PEAK_TFLOPS * 1e12), 4),
        "factorised_weights_per_s": round(args.steps * weights / elapsed, 1),
        "flops_per_step": F,
        "roofline": {
            "kernel": "gemm_nt_kernel<kEpiRhs> (R = Wt V + rho (Z - Lam), V read as V^T)",
            "note": ("timed as it runs in the pipeline, beside the Cholesky chain (for r_p <= "
                     "2048 on 7 of the 8 XCDs, yielding issue cycles to the chain); averaged over "
                     "every RHS launch of the timed steps; the same kernel alone on the whole "
                     "chip: see the standalone kernel profile"),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": FP32_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / FP32_MFMA_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(rhs_avg_s * 1e3, 4),
            "launches": rhs_n,
            "flops_per_launch": rhs_flops / max(rhs_n, 1),
        },
        "svid_update_standalone": svid if not single else svid[next(iter(svid))],
        "bpw": round(bits / weights, 4),
        "bpw_with_fp16_scales": round((bits + scale_bits) / weights, 4),
        "rel_err_wtilde": (stats_all[0]["rel_err_wtilde"] if single
                           else [s["rel_err_wtilde"] for s in stats_all]),
        "rel_err_w": (stats_all[0]["rel_err_w"] if single
                      else [s["rel_err_w"] for s in stats_all]),
    }
    if single:
        m, n, r, iters = wl0.m, wl0.n, wl0.r, runs[0][1]
        phases = phases_all[0]
        line["flops_per_iter"] = flops_per_iter(m, n, r)
        # from one untimed run with every phase timed (the chain phase is the
        # Gram plus the Cholesky chain; phases of different streams overlap)
        line["phase_ms_per_iter"] = {p: round(phases[p][0] / max(iters, 1), 4)
                                     for p in ("gemm_rhs", "gemm_solve", "chain", "svid")}
        line["phase_ms_per_step"] = {p: round(phases[p][0], 3) for p in ("prep", "finish")}
        line["phase_source"] = "one untimed run with every phase timed"
        sol_s = phases["gemm_solve"][0] / max(phases["gemm_solve"][1], 1) / 1e3
        # the solve GEMM runs alone on the chip, on the critical path; its
        # launches alternate between the U-half (m rows) and the V-half (n
        # rows), 2 rows r^2 flops each
        sol_f = (m + n) * r * r
        line["solve_gemm"] = {
            "flops_per_launch": sol_f,
            "avg_launch_ms": round(sol_s * 1e3, 4),
            "tflops": round(sol_f / sol_s / 1e12, 2),
            "frac_of_peak": round(sol_f / sol_s / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
            "source": "the untimed run with every phase timed (mean over U- and V-half launches)",
        }
    return line


if __name__ == "__main__":
    main()
