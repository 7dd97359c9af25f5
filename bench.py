#!/usr/bin/env python3
"""Throughput of the GEMM-epilogue training step on one MI355X.

Workload (the step that is timed): one SGD-momentum training step of the
784-2048-2048-10 ReLU MLP, FP16 storage with FP32 accumulation and FP32
master weights, batch 4096, lr 0.05, momentum 0.9, on the seeded
template-plus-noise images; the 50 batches of the run are resident in HBM
before timing starts.  A step is forward (3 GEMMs with bias/ReLU epilogues),
softmax cross-entropy forward/backward, the TN weight-gradient GEMMs, column
sums, the masked NT dgrad GEMMs and one flat momentum update, all in
libgemm_epilogue.so.

Printed: one JSON line (stdout) with samples/s, the roofline of the dominant
kernel (the NN GEMM-epilogue kernel, timed with HIP events on its stream),
the standalone 4096^3 GEMM-epilogue rates of the three layouts, and the
oracle's CPU throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2500.0   # MI355X dense FP16/BF16 MFMA
# HBM bytes per launch of the roofline kernel (the fwd2 launch below):
# FETCH_SIZE + WRITE_SIZE counter passes of rocprofv3 over this script, scaled
# by the counters' reading for a plain copy of known size (--copy-calibration),
# as listed in profiles/mlp784-2048-2048-10_fp16_b4096_hbm_bytes.md.  Taken on
# the current kernel; to be re-measured whenever the kernel changes.
NN_TRAFFIC_BYTES = 101.24e6
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
DIMS = [784, 2048, 2048, 10]
BATCH, LR, MU, N_BATCHES = 4096, 0.05, 0.9, 50


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def mlp_flops_per_sample(dims):
    """Forward 2*sum(d_in*d_out), weight gradients the same, dgrad for layers 2..L."""
    f = sum(2 * a * b for a, b in zip(dims[:-1], dims[1:]))
    dg = sum(2 * a * b for a, b in zip(dims[1:-1], dims[2:]))
    return 2 * f + dg


def event_time_ms(torch, fn, iters):
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for i in range(iters):
        fn(i)
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1)


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
    return {"value": n / dt, "unit": "samples/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} oracle steps of batch 512 of the same 784-2048-2048-10 FP16-storage "
                      f"workload ({n} samples, {dt:.1f} s, float64 numpy)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm4096", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB elementwise copy, the reference dispatch for "
                         "scaling hardware byte counters (FETCH_SIZE / WRITE_SIZE) to bytes")
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
    K, W = args.steps, args.warmup

    # ---- resident inputs: the run's batches, parameters, buffers ----------
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
    ms = event_time_ms(torch, lambda i: step(W + i), K)
    torch.cuda.synchronize()
    ms_per_step = ms / K
    samples_per_s = BATCH * K / (ms / 1e3)
    flops_step = mlp_flops_per_sample(DIMS) * BATCH
    loss = float(tr.loss.item())

    # ---- dominant kernel: the 256x128 four-wave GEMM-epilogue kernel, which
    # runs the step's two 4096x2048x2048 GEMMs (forward fwd2 and the masked
    # dgrad); its forward launch (H2 = relu(H1 W2 + b2)) is replayed with the
    # step's own operands on the same stream and timed with HIP events.
    views = tr.workspace_views(BATCH)
    H1, H2 = views["H"]
    lowp = tr.params_lowp
    o1 = 784 * 2048 + 2048
    W2 = lowp[o1:o1 + 2048 * 2048].view(2048, 2048)
    b2 = tr.params[o1 + 2048 * 2048:o1 + 2048 * 2048 + 2048]
    f_nn = 2 * BATCH * 2048 * 2048

    def fwd2(i):
        ge.gemm_bias_act(H1, W2, "NN", bias=b2, act="relu", out=H2)

    for i in range(3):
        fwd2(i)
    nn_ms = event_time_ms(torch, fwd2, K) / K
    nn_tflops = f_nn / (nn_ms / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(nn_tflops, 1), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(nn_tflops / PEAK_F16_TFLOPS, 4),
                "traffic": NN_TRAFFIC_BYTES,
                "kernel": "gemm_w4_kernel<f16, NN, 256x128 tile> (fwd2 of the step, 4096x2048x2048)",
                "avg_launch_us": round(nn_ms * 1e3, 2)}

    # ---- standalone 4096^3 GEMM + bias + ReLU epilogue, three layouts ------
    gemm4096 = None
    if not args.no_gemm4096:
        gemm4096 = {}
        M = N = Kd = 4096
        g = torch.Generator(device="cpu").manual_seed(1)
        for layout in ("NN", "NT", "TN"):
            sa = (M, Kd) if layout != "TN" else (Kd, M)
            sb = (Kd, N) if layout != "NT" else (N, Kd)
            A = (torch.randn(sa, generator=g) / 64).half().to(dev)
            Bm = (torch.randn(sb, generator=g) / 64).half().to(dev)
            bias = (torch.randn(N, generator=g) * 0.1).to(dev)
            out = torch.empty(M, N, dtype=torch.float16, device=dev)
            run = lambda i: ge.gemm_bias_act(A, Bm, layout, bias=bias, act="relu", out=out)
            for i in range(3):
                run(i)
            t = event_time_ms(torch, run, 20) / 20
            tf = 2 * M * N * Kd / (t / 1e3) / 1e12
            gemm4096[layout] = {"us": round(t * 1e3, 1), "tflops": round(tf, 1),
                                "frac_of_peak": round(tf / PEAK_F16_TFLOPS, 4)}
            del A, Bm, out

    if args.copy_calibration:
        # reads 256 MiB and writes 256 MiB; run it twice so one dispatch is warm
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        cpu = cpu_baseline()

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
        "step_tflops": round(flops_step / (ms_per_step / 1e3) / 1e12, 1),
        "final_loss": round(loss, 6),
        "roofline": roofline,
        "gemm_epilogue_4096": gemm4096,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
