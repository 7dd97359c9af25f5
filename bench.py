#!/usr/bin/env python3
"""Throughput of the GEMM-epilogue training path on one MI355X.

Headline workload (the timed step): one SGD-momentum training step of the
784-2048-2048-10 ReLU MLP, FP16 storage with FP32 accumulation and FP32 master
weights, batch 4096, lr 0.05, momentum 0.9, on the seeded template-plus-noise
images; the 50 batches of the run are resident in HBM before timing starts.
A step is the forward GEMMs with bias/ReLU epilogues, the fused output layer
(logits, softmax cross-entropy, dZ, bias gradient, masked dgrad), the TN
weight-gradient GEMMs, the masked NT dgrad GEMM and one flat momentum update,
all in libgemm_epilogue.so.

Printed: one JSON line (stdout) with samples/s of that step, the roofline of
its dominant kernel (timed live with HIP events on its stream), and beside it
every other configuration of the path -- the 784-256-10 FP32 epoch (with and
without hipGraph capture), the standalone 4096^3 GEMM-epilogue in three
layouts, the transformer MLP block forward+backward, the GRU LM step, the
bandwidth-bound kernels with the Infinity Cache flushed -- each a median with
its coefficient of variation, the shader clock measured under MFMA load, and
the oracle's CPU throughput on a bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2500.0   # MI355X dense FP16/BF16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
NOMINAL_GHZ = 2.4          # the clock the dense peak is quoted at
DIMS = [784, 2048, 2048, 10]
BATCH, LR, MU, N_BATCHES = 4096, 0.05, 0.9, 50

# HBM bytes per launch of the roofline kernel (the fwd2 launch below), from the
# FETCH_SIZE and WRITE_SIZE counter passes of rocprofv3 over this script,
# scaled by the counters' reading for a plain copy of known size (run with
# --copy-calibration; the factors are listed with the counts under profiles/).
# Keyed by the SHA-256 of the GEMM kernel sources they were measured on: when
# the sources change, the figure no longer describes the kernel and `traffic`
# is reported as null until the counters are taken again.
TRAFFIC_BY_SOURCE = {
    # FETCH_SIZE 41,124 KiB x 2.0 + WRITE_SIZE 16,384 KiB x 1.0 per launch
    "5515feea01e13e03": 100_999_168,
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_source_sha() -> str:
    h = hashlib.sha256()
    for f in ("gemm_kernel.h", "gemm.hip"):
        with open(os.path.join(ROOT, "gemm_epilogue_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def mlp_flops_per_sample(dims):
    """Forward 2*sum(d_in*d_out), weight gradients the same, dgrad for layers 2..L."""
    f = sum(2 * a * b for a, b in zip(dims[:-1], dims[1:]))
    dg = sum(2 * a * b for a, b in zip(dims[1:-1], dims[2:]))
    return 2 * f + dg


def stats(xs):
    xs = np.asarray(xs, dtype=np.float64)
    return float(np.median(xs)), float(xs.std() / xs.mean()) if xs.size > 1 and xs.mean() > 0 else 0.0


class Timer:
    """HIP events on torch's current stream (the stream every library call
    enqueues on)."""

    def __init__(self, torch):
        self.torch = torch

    def once(self, fn):
        t = self.torch
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3  # us

    def per_launch(self, fn, reps=10, n=20, warm=3, warm_ms=30.0):
        """Median and CV over `reps` measurements of `n` back-to-back launches
        each (the host enqueues faster than the kernels run, so no host time
        enters the interval).  The untimed warm-up keeps the GPU busy for at
        least `warm_ms` first: straight after the host-side set-up of a new
        workload the first few milliseconds of launches ran up to 8 % slower
        (4096^3 GEMM: 128-130 us against 120 us once warm)."""
        for _ in range(warm):
            fn()
        self.torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < warm_ms:
            for _ in range(n):
                fn()
            self.torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            ts.append(self.once(lambda: [fn() for _ in range(n)]) / n)
        return stats(ts)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds_target=12.0):
    """The oracle's MLP step on host cores over a bounded sample (batches of 512)."""
    import threadpoolctl
    import datagen
    import oracle
    p = datagen.he_uniform_flat(DIMS)
    v = np.zeros_like(p)
    n, t0, reps = 0, time.perf_counter(), 0
    while True:
        X, y = datagen.template_images(512, 200, fmt="f16", batch=1000 + reps)
        out = oracle.mlp_step(p, v, DIMS, X, y, LR, MU, plan="f16")
        p, v = out["params"], out["vel"]
        n += X.shape[0]
        reps += 1
        if time.perf_counter() - t0 >= seconds_target or reps >= 40:
            break
    dt = time.perf_counter() - t0
    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info] or [1])
    return {"value": round(n / dt, 1), "unit": "samples/s", "cores": cores, "kind": "oracle",
            "cpu": cpu_model(), "host_threads": os.cpu_count(),
            "sample": f"{reps} oracle steps of batch 512 of the same 784-2048-2048-10 FP16-storage "
                      f"workload ({n} samples, {dt:.1f} s, float64 numpy, {cores} BLAS threads)",
            "single_thread": cpu_single_thread()}


def cpu_single_thread(reps=10):
    """The oracle on one host thread for the two small workloads: one step of
    the 784-256-10 FP32 MLP at batch 128 and one 128x256x784 FP16 GEMM with
    bias + ReLU (median of `reps` calls each)."""
    import threadpoolctl
    import datagen
    import oracle
    dims = [784, 256, 10]
    p = datagen.he_uniform_flat(dims)
    v = np.zeros_like(p)
    X, y = datagen.template_images(128, 100, fmt="f32", batch=2000)
    A, B, bias = datagen.gemm_operands(128, 256, 784, "NN", seed=3)
    out = {}
    with threadpoolctl.threadpool_limits(1):
        for name, fn in (("mlp_784_256_10_step_b128_us",
                          lambda: oracle.mlp_step(p, v, dims, X, y, 0.05, 0.9, plan="f32")),
                         ("gemm_128x256x784_bias_relu_us",
                          lambda: oracle.gemm_epilogue(A, B, "NN", bias=bias, act="relu", out_fmt="f16"))):
            ts = []
            for _ in range(reps):
                t0 = time.perf_counter()
                fn()
                ts.append((time.perf_counter() - t0) * 1e6)
            out[name] = round(float(np.median(ts)), 1)
    out["threads"] = 1
    return out


def measure_clock(torch, ge, dev):
    """Shader clock under MFMA load on all CUs (library probe)."""
    blocks = 1024
    ticks = torch.zeros(3 * blocks, dtype=torch.int64, device=dev)
    lib = ge.lib
    ge._lib.check(lib.ge_clock_probe(ctypes.c_void_p(ticks.data_ptr()), blocks, 4000,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)), "ge_clock_probe")
    torch.cuda.synchronize()
    t = ticks.view(blocks, 3).cpu().numpy().astype(np.float64)
    ghz = t[:, 0] / (t[:, 1] / 100e6) / 1e9
    return round(float(np.median(ghz)), 3)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="headline step and roofline only")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB elementwise copy, the reference dispatch for "
                         "scaling hardware byte counters (FETCH_SIZE / WRITE_SIZE) to bytes")
    ap.add_argument("--only", choices=("gemm4096", "gemm_small", "cfg0", "block", "gru", "bandwidth", "blas"),
                    help="time one of the extra workloads alone and print its record (for profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build runs the path on a single MI355X "
              "(see the sharding notes); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import datagen
    import gemm_epilogue_amd as ge

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tm = Timer(torch)
    K, W = args.steps, args.warmup

    if args.only:
        runs = {"gemm4096": lambda: bench_gemm4096(torch, ge, dev, tm),
                "gemm_small": lambda: bench_gemm_small(torch, ge, dev, tm),
                "cfg0": lambda: bench_cfg0(torch, ge, datagen, dev, tm),
                "block": lambda: bench_block(torch, ge, datagen, dev, tm),
                "gru": lambda: bench_gru(torch, ge, datagen, dev, tm),
                "bandwidth": lambda: bench_bandwidth(torch, ge, datagen, dev, tm),
                "blas": lambda: bench_blas_context(torch, ge, dev, tm)}
        print(json.dumps({"only": args.only, args.only: runs[args.only]()}), flush=True)
        return

    # ---- headline: the 784-2048-2048-10 FP16 training step ---------------
    log("generating inputs")
    nb = min(N_BATCHES, max(1, K + W))
    Xs, ys = [], []
    for b in range(nb):
        X, y = datagen.template_images(BATCH, 200, fmt="f16", batch=b)
        Xs.append(torch.from_numpy(X).to(torch.float16).to(dev))
        ys.append(torch.from_numpy(y).to(dev))
    p0 = torch.from_numpy(datagen.he_uniform_flat(DIMS)).float().to(dev)
    tr = ge.MLPTrainer(DIMS, BATCH, torch.float16, params=p0)

    def step(i):
        tr.step(Xs[i % nb], ys[i % nb], LR, MU)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    log("timing steps")
    # K steps bracketed by events (the value), with an event after every step
    # for the per-step median and CV
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(K):
        step(W + i)
        evs[i + 1].record()
    evs[-1].synchronize()
    torch.cuda.synchronize()
    total_ms = evs[0].elapsed_time(evs[-1])
    per_step_us = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(K)]
    ms_per_step = total_ms / K
    samples_per_s = BATCH * K / (total_ms / 1e3)
    flops_step = mlp_flops_per_sample(DIMS) * BATCH
    loss = float(tr.loss.item())
    step_med, step_cv = stats(per_step_us)
    n0 = ge.lib.ge_launch_count()
    step(0)
    launches_cfg2 = int(ge.lib.ge_launch_count() - n0)
    torch.cuda.synchronize()

    # ---- roofline: the dominant kernel of the step -------------------------
    # the eight-wave 256x128 GEMM-epilogue kernel runs the step's two
    # 4096x2048x2048 GEMMs (forward H2 = relu(H1 W2 + b2) and the masked
    # dgrad); its forward launch is replayed with the step's own operands
    views = tr.workspace_views(BATCH)
    H1, H2 = views["H"]
    lowp = tr.params_lowp
    o1 = 784 * 2048 + 2048
    W2 = lowp[o1:o1 + 2048 * 2048].view(2048, 2048)
    b2 = tr.params[o1 + 2048 * 2048:o1 + 2048 * 2048 + 2048]
    f_nn = 2 * BATCH * 2048 * 2048
    nn_us, nn_cv = tm.per_launch(lambda: ge.gemm_bias_act(H1, W2, "NN", bias=b2, act="relu", out=H2),
                                 reps=10, n=20)
    nn_tflops = f_nn / (nn_us * 1e-6) / 1e12
    clock = measure_clock(torch, ge, dev)
    sha = gemm_source_sha()
    roofline = {"bound": "mfma", "achieved": round(nn_tflops, 1), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(nn_tflops / PEAK_F16_TFLOPS, 4),
                "traffic": TRAFFIC_BY_SOURCE.get(sha),
                "kernel": "gemm_x8_kernel<f16, NN, 256x128 tile> (fwd2 of the step, 4096x2048x2048)",
                "avg_launch_us": round(nn_us, 2), "launch_cv": round(nn_cv, 4),
                "algorithmic_flop": f_nn, "gemm_source_sha": sha,
                "measured_clock_ghz": clock,
                "frac_at_measured_clock": round(nn_tflops / (PEAK_F16_TFLOPS * clock / NOMINAL_GHZ), 4)}

    rec = {
        "metric": "train-step samples/s + GEMM-epilogue TFLOP/s (% MFMA peak), 1 MI355X",
        "value": round(samples_per_s, 1),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "mlp-784-2048-2048-10 train step, fp16 storage, fp32 accumulation, "
                               "batch 4096, sgd-momentum lr 0.05 mu 0.9",
                   "global_batch": BATCH, "layers": DIMS, "parallelism": "single-gpu"},
        "step_us_median": round(step_med, 2),
        "step_cv": round(step_cv, 4),
        "step_tflops": round(flops_step / (ms_per_step / 1e3) / 1e12, 1),
        "launches_per_step": launches_cfg2,
        "final_loss": round(loss, 6),
        "roofline": roofline,
    }
    del Xs, ys, tr
    torch.cuda.empty_cache()

    if not args.no_extra:
        # each workload starts from an empty allocator cache, in this order:
        # measured in the same process after the block and the 784-256-10
        # epochs, the GRU step's memory-bound kernels ran up to twice as long
        # (4.4 ms against 3.7 ms alone), and the 4096^3 GEMMs after the GRU
        # step 12 % longer; here each lands within a few per cent of its
        # own process
        def fresh(fn):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            return fn()
        rec["gemm_epilogue_4096"] = fresh(lambda: bench_gemm4096(torch, ge, dev, tm))
        rec["gru_lm_step"] = fresh(lambda: bench_gru(torch, ge, datagen, dev, tm))
        rec["mlp_784_256_10_epoch"] = fresh(lambda: bench_cfg0(torch, ge, datagen, dev, tm))
        rec["mlp_block"] = fresh(lambda: bench_block(torch, ge, datagen, dev, tm))
        rec["bandwidth_kernels"] = fresh(lambda: bench_bandwidth(torch, ge, datagen, dev, tm))
        # after the others: timed right before the GRU step it left that
        # step's memory-bound kernels slower (4.4 against 3.7 ms)
        rec["gemm_epilogue_128x256x784"] = fresh(lambda: bench_gemm_small(torch, ge, dev, tm))
        rec["blas_context"] = fresh(lambda: bench_blas_context(torch, ge, dev, tm))

    if args.copy_calibration:
        # reads 256 MiB and writes 256 MiB; run it twice so one dispatch is warm
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        rec["cpu_baseline"] = cpu_baseline()
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def bench_gemm4096(torch, ge, dev, tm):
    """Standalone 4096^3 GEMM + bias + ReLU epilogue, FP16 inputs, three layouts,
    FP16 and FP32 stores: median of 10 x 20 back-to-back launches."""
    log("timing the 4096^3 GEMM epilogue")
    out = {}
    M = N = Kd = 4096
    g = torch.Generator(device="cpu").manual_seed(1)
    for layout in ("NN", "NT", "TN"):
        sa = (M, Kd) if layout != "TN" else (Kd, M)
        sb = (Kd, N) if layout != "NT" else (N, Kd)
        A = (torch.randn(sa, generator=g) / 64).half().to(dev)
        Bm = (torch.randn(sb, generator=g) / 64).half().to(dev)
        bias = (torch.randn(N, generator=g) * 0.1).to(dev)
        r = {}
        for store, dt in (("f16", torch.float16), ("f32", torch.float32)):
            C = torch.empty(M, N, dtype=dt, device=dev)
            us, cv = tm.per_launch(lambda: ge.gemm_bias_act(A, Bm, layout, bias=bias, act="relu", out=C))
            tf = 2 * M * N * Kd / (us * 1e-6) / 1e12
            r[store] = {"us": round(us, 1), "cv": round(cv, 4), "tflops": round(tf, 1),
                        "frac_of_peak": round(tf / PEAK_F16_TFLOPS, 4)}
            del C
        out[layout] = r
        del A, Bm
    torch.cuda.empty_cache()
    return out


def bench_gemm_small(torch, ge, dev, tm):
    """The small GEMM-epilogue shape, 128x256x784 (one 784-wide layer on a
    128-row batch): A, B ~ N(0, 1/sqrt(K)) in FP16, bias + ReLU, three layouts,
    FP16 and FP32 stores.  Latency-bound (51.4 MFLOP per launch): reported as
    the GPU's time per launch within a captured graph, and the time per eager
    call, each a median of 10 repetitions."""
    log("timing the 128x256x784 GEMM epilogue")
    out = {}
    M, N, Kd = 128, 256, 784
    g = torch.Generator(device="cpu").manual_seed(3)
    for layout in ("NN", "NT", "TN"):
        sa = (M, Kd) if layout != "TN" else (Kd, M)
        sb = (Kd, N) if layout != "NT" else (N, Kd)
        A = (torch.randn(sa, generator=g) / Kd ** 0.5).half().to(dev)
        Bm = (torch.randn(sb, generator=g) / Kd ** 0.5).half().to(dev)
        bias = (torch.randn(N, generator=g) * 0.1).to(dev)
        r = {}
        for store, dt in (("f16", torch.float16), ("f32", torch.float32)):
            C = torch.empty(M, N, dtype=dt, device=dev)
            fn = lambda: ge.gemm_bias_act(A, Bm, layout, bias=bias, act="relu", out=C)
            # eager calls are bound by the host at this size; 20 launches
            # captured in one graph give the GPU's own time per launch
            eager_us, eager_cv = tm.per_launch(fn)
            us, cv = graph_per_launch(torch, tm, fn)
            r[store] = {"us": round(us, 2), "cv": round(cv, 4),
                        "tflops": round(2 * M * N * Kd / (us * 1e-6) / 1e12, 2),
                        "eager_us": round(eager_us, 2), "eager_cv": round(eager_cv, 4)}
        out[layout] = r
    return out


def graph_per_launch(torch, tm, fn, n=20):
    """Time per launch of `fn` with `n` launches captured in one graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    torch.cuda.synchronize()
    us, cv = tm.per_launch(g.replay, reps=10, n=5)
    del g
    return us / n, cv


def bench_blas_context(torch, ge, dev, tm):
    """Context, not part of the path: the platform BLAS (torch.matmul) on the
    step's forward GEMM shapes and on 4096^3, FP16 NN with an FP16 store and
    no epilogue, beside this library's kernel on the same operands, plain and
    with the bias + ReLU epilogue.  Median of 10 x 20 back-to-back launches."""
    log("timing the platform BLAS for context")
    out = {}
    g = torch.Generator(device="cpu").manual_seed(2)
    for (M, N, Kd) in ((4096, 2048, 2048), (4096, 2048, 784), (4096, 4096, 4096)):
        A = (torch.randn(M, Kd, generator=g) / 64).half().to(dev)
        Bm = (torch.randn(Kd, N, generator=g) / 64).half().to(dev)
        bias = (torch.randn(N, generator=g) * 0.1).to(dev)
        C = torch.empty(M, N, dtype=torch.float16, device=dev)
        fl = 2 * M * N * Kd
        r = {}
        for name, fn in (("blas_matmul", lambda: torch.matmul(A, Bm, out=C)),
                         ("ours_plain", lambda: ge.gemm_bias_act(A, Bm, "NN", out=C)),
                         ("ours_bias_relu", lambda: ge.gemm_bias_act(A, Bm, "NN", bias=bias, act="relu", out=C))):
            us, cv = tm.per_launch(fn)
            r[name] = {"us": round(us, 1), "cv": round(cv, 4),
                       "frac_of_peak": round(fl / (us * 1e-6) / 1e12 / PEAK_F16_TFLOPS, 4)}
        out[f"{M}x{N}x{Kd}"] = r
        del A, Bm, bias, C
    torch.cuda.empty_cache()
    return out


def bench_cfg0(torch, ge, datagen, dev, tm):
    """784-256-10 FP32, batch 128 (46 batches + 112), lr 0.1, momentum 0.9: one
    warm-up epoch, then 11 epochs each from the same initial weights and zero
    velocity, timed per epoch, for the one-launch persistent step (the
    default plan) and for the launch chain; the chain's epoch is also captured
    once as a hipGraph and replayed 11 times (the capstone's launch-overhead
    question)."""
    log("timing the 784-256-10 epoch")
    dims = datagen.mlp_dims_cfg0()
    Xall, yall = datagen.template_images(6000, 100, fmt="f32")
    tX = torch.from_numpy(Xall).float().to(dev)
    ty = torch.from_numpy(yall).to(dev)
    p0 = torch.from_numpy(datagen.he_uniform_flat(dims)).float().to(dev)
    batches = [(s, min(6000, s + 128)) for s in range(0, 6000, 128)]

    def run(plan, graph_too):
        tr = ge.MLPTrainer(dims, 128, torch.float32, params=p0, plan=plan)

        def epoch():
            for s, e in batches:
                tr.step(tX[s:e], ty[s:e], 0.1, 0.9)

        def reset():
            tr.params.copy_(p0)
            tr.velocity.zero_()

        n0 = ge.lib.ge_launch_count()
        tr.step(tX[:128], ty[:128], 0.1, 0.9)
        launches = int(ge.lib.ge_launch_count() - n0)
        n0 = ge.lib.ge_launch_count()
        tr.step(tX[5888:], ty[5888:], 0.1, 0.9)
        launches_last = int(ge.lib.ge_launch_count() - n0)
        reset()
        epoch()  # warm-up epoch
        ts = []
        for _ in range(11):
            reset()
            ts.append(tm.once(epoch))
        eager_us, eager_cv = stats(ts)
        reset()
        epoch()
        torch.cuda.synchronize()
        p_eager = tr.params.clone()
        out = {"samples_per_s": round(6000 / (eager_us * 1e-6), 1), "epoch_us": round(eager_us, 1),
               "epoch_cv": round(eager_cv, 4), "us_per_step": round(eager_us / len(batches), 2),
               "launches_per_step": launches, "launches_last_step": launches_last}
        if graph_too:
            # one captured graph holds the whole epoch (47 steps)
            reset()
            graph = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                epoch()  # the capture stream's own warm-up
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(graph):
                epoch()
            reset()
            graph.replay()
            torch.cuda.synchronize()
            gts = []
            for _ in range(11):
                reset()
                gts.append(tm.once(graph.replay))
            graph_us, graph_cv = stats(gts)
            # the graph's epoch must land where the eager one does
            reset()
            graph.replay()
            torch.cuda.synchronize()
            out["graph"] = {"samples_per_s": round(6000 / (graph_us * 1e-6), 1), "epoch_us": round(graph_us, 1),
                            "epoch_cv": round(graph_cv, 4), "same_params_as_eager": bool(torch.equal(p_eager, tr.params))}
            del graph
        del tr
        return out, p_eager

    pers, p_pers = run("persistent", False)
    chain, p_chain = run("chain", True)
    d = (p_pers - p_chain).abs().max().item()
    res = dict(pers)
    res.update({"plan": "persistent", "steps": len(batches), "chain": chain,
                "params_max_abs_diff_persistent_vs_chain": d, "flop_per_epoch": 4.909e9,
                "note": "median of 11 epochs after a warm-up epoch, each from the initial weights"})
    return res


def bench_block(torch, ge, datagen, dev, tm):
    """Transformer MLP block forward+backward, 98,304 x 512, hidden 1536, BF16."""
    log("timing the MLP block")
    R, D, F = 98304, 512, 1536
    x, wu, wd, dy = datagen.block_inputs(R, D, F, seed=3)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(dev)
    tx, twu, twd, tdy = t(x), t(wu), t(wd), t(dy)
    del x, wu, wd, dy
    o = ge.mlp_block_fwd_bwd(tx, twu, twd, tdy, eps=1e-6, slope=0.5)
    us, cv = tm.per_launch(lambda: ge.mlp_block_fwd_bwd(tx, twu, twd, tdy, eps=1e-6, slope=0.5, out=o,
                                                        workspace=o["workspace"]), reps=10, n=3, warm=2)
    flop = 6 * 2 * R * D * F
    n0 = ge.lib.ge_launch_count()
    ge.mlp_block_fwd_bwd(tx, twu, twd, tdy, eps=1e-6, slope=0.5, out=o, workspace=o["workspace"])
    launches = int(ge.lib.ge_launch_count() - n0)
    torch.cuda.synchronize()
    # the forward alone, A/B: the chain's three launches (RMSNorm; up projection
    # with the LeakyReLU^2 epilogue and the pre-activation store; down
    # projection with the residual) against the one-kernel forward, storing y
    # only and storing what the backward pass reads (r, n, u) as well
    fflop = 2 * 2 * R * D * F
    y2 = torch.empty_like(o["y"])
    fwd = {}

    def chain_fwd():
        ge.rmsnorm_fwd(tx, 1e-6, y=o["n"], r=o["r"])
        ge.gemm_bias_act(o["n"], twu, "NN", out=o["a"], act="lrelu_sq", slope=0.5, pre=o["u"])
        ge.gemm_bias_act(o["a"], twd, "NN", out=o["y"], residual=tx)

    ws = torch.empty(int(ge.lib.mlp_block_fused_workspace_bytes(D, F)), dtype=torch.uint8, device=dev)
    runs = {"chain": chain_fwd,
            "fused_y_only": lambda: ge.mlp_block_fwd_fused(tx, twu, twd, y=y2, workspace=ws),
            "fused_with_r_n_u": lambda: ge.mlp_block_fwd_fused(tx, twu, twd, y=y2, r=o["r"], n=o["n"], u=o["u"],
                                                               workspace=ws)}
    for name, fn in runs.items():
        fus, fcv = tm.per_launch(fn, reps=10, n=5, warm=2)
        fwd[name] = {"us": round(fus, 1), "cv": round(fcv, 4), "tokens_per_s": round(R / (fus * 1e-6), 1),
                     "tflops": round(fflop / (fus * 1e-6) / 1e12, 1)}
    torch.cuda.synchronize()
    fwd["fused_vs_chain_y_cos"] = float(torch.nn.functional.cosine_similarity(
        y2.float().flatten(), o["y"].float().flatten(), dim=0))
    del o, tx, twu, twd, tdy, y2, ws
    torch.cuda.empty_cache()
    return {"tokens_per_s": round(R / (us * 1e-6), 1), "us": round(us, 1), "cv": round(cv, 4),
            "tflops": round(flop / (us * 1e-6) / 1e12, 1), "frac_of_peak": round(flop / (us * 1e-6) / 1e12 /
                                                                             PEAK_F16_TFLOPS, 4),
            "launches": launches, "flop": flop, "forward_ab": fwd, "forward_flop": fflop}


def bench_gru(torch, ge, datagen, dev, tm):
    """GRU byte LM training step: V 256, H 1024, batch 64, T 128, lr 0.01,
    momentum 0.9; the recurrence as one persistent launch per direction (the
    default) and as one GEMM and one gate launch per timestep."""
    log("timing the GRU LM step")
    V, H, B, T = 256, 1024, 64, 128
    P = datagen.gru_params(H, V)
    order = ("E", "W_i", "b_i", "W_h", "b_h", "W_c", "b_c")
    flat = torch.from_numpy(np.concatenate([np.asarray(P[k], np.float64).ravel() for k in order])).float().to(dev)
    tok = torch.from_numpy(datagen.zipf_tokens(B, T + 1, seed=B + T, vocab=V)).to(dev)
    flop = 6 * 2 * B * T * H * 3 * H + 3 * 2 * B * T * H * V
    out = {}
    for mode in ("persistent", "stepwise"):
        tr = ge.GRUTrainer(V, H, B, T, eps=1e-6, params=flat, recurrence=mode)
        us, cv = tm.per_launch(lambda: tr.step(tok, 0.01, 0.9), reps=10, n=3, warm=2)
        n0 = ge.lib.ge_launch_count()
        tr.step(tok, 0.01, 0.9)
        launches = int(ge.lib.ge_launch_count() - n0)
        torch.cuda.synchronize()
        out[mode] = {"tokens_per_s": round(B * T / (us * 1e-6), 1), "us": round(us, 1), "cv": round(cv, 4),
                     "tflops": round(flop / (us * 1e-6) / 1e12, 1), "launches": launches}
        del tr
    out["flop"] = flop
    out["tokens_per_s"] = out["persistent"]["tokens_per_s"]
    return out


def bench_bandwidth(torch, ge, datagen, dev, tm):
    """HBM-bound kernels.  Cold: back-to-back launches rotating over enough
    copies of the operands (> 512 MB together) that every launch reads data the
    256 MB Infinity Cache no longer holds.  Warm: the same operands every launch."""
    log("timing the bandwidth-bound kernels")
    out = {}

    def entry(name, nbytes, fns):
        c_us, c_cv = tm.per_launch(lambda it=iter(range(1 << 30)): fns[next(it) % len(fns)](),
                                   reps=10, n=4 * len(fns))
        w_us, w_cv = tm.per_launch(fns[0], reps=10, n=20)
        out[name] = {"bytes": nbytes, "copies_rotated": len(fns),
                     "cold": {"us": round(c_us, 2), "cv": round(c_cv, 4), "gbs": round(nbytes / c_us / 1e3, 1),
                              "frac_of_hbm": round(nbytes / c_us / 1e3 / PEAK_HBM_GBS, 4)},
                     "warm": {"us": round(w_us, 2), "cv": round(w_cv, 4), "gbs": round(nbytes / w_us / 1e3, 1),
                              "frac_of_hbm": round(nbytes / w_us / 1e3 / PEAK_HBM_GBS, 4)}}

    def copies(nbytes):
        return max(2, -(-(600 << 20) // nbytes))

    nb = 4096 * 4096 * 4 + 4096 * 4
    Xs = [torch.randn(4096, 4096, device=dev) for _ in range(copies(nb))]
    cs = torch.empty(4096, device=dev)
    ws = torch.empty(max(1, int(ge.lib.colsum_workspace_bytes(4096, 4096))), dtype=torch.uint8, device=dev)
    entry("colsum_f32_4096x4096", nb, [lambda X=X: ge.colsum(X, out=cs, workspace=ws) for X in Xs])
    del Xs
    R, D = 98304, 512
    nb = R * D * 2 * 2 + R * 4
    xs = [torch.randn(R, D, device=dev).to(torch.bfloat16) for _ in range(copies(nb))]
    ys = [torch.empty_like(x) for x in xs]
    r = torch.empty(R, device=dev)
    entry("rmsnorm_fwd_bf16_98304x512", nb,
          [lambda x=x, y=y: ge.rmsnorm_fwd(x, 1e-6, y=y, r=r) for x, y in zip(xs, ys)])
    del ys
    nb = R * D * (2 + 4 + 2 + 2) + R * 4
    n = copies(nb)
    dns = [torch.randn(R, D, device=dev) for _ in range(n)]
    dress = [torch.randn(R, D, device=dev).to(torch.bfloat16) for _ in range(n)]
    dxs = [torch.empty_like(xs[0]) for _ in range(n)]
    entry("rmsnorm_bwd_bf16_98304x512", nb,
          [lambda i=i: ge.rmsnorm_bwd(xs[i % len(xs)], r, dns[i], dres=dress[i], dx=dxs[i]) for i in range(n)])
    del xs, dns, dress, dxs
    P = 5824522
    nb = P * 22
    n = copies(nb)
    sets = [(torch.randn(P, device=dev) * 0.05, torch.randn(P, device=dev) * 0.01, torch.zeros(P, device=dev),
             torch.empty(P, dtype=torch.float16, device=dev)) for _ in range(n)]
    entry("sgd_momentum_f32_5824522_with_f16_copy", nb,
          [lambda s=s: ge.sgd_momentum(s[0], s[1], s[2], 0.0, 0.0, s[3]) for s in sets])
    del sets
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
