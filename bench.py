#!/usr/bin/env python3
"""Benchmark of the W2A8 ternary decode product on one MI355X.

One step = one pass of the decode hot path over one batch: per-token int8
quantisation of the bf16 activations (bitnet_quant_act) followed by the W2A8
product (bitnet_w2a8_gemv), for the 13824x2560 fused gate+up shape at batch 1
(weights from absmean-ternarised N(0, 0.02), activations N(0,1) bf16).  Every
step reads a different copy of the packed weights, from a rotation larger than
twice the 256 MB last-level cache, so the weight stream comes from HBM.

value = packed-weight bytes (N*K/4) per step / step time, in GB/s.
The roofline object prices the product kernel against 8 TB/s using its
algorithmic bytes (packed weights + fp32 block scales + int8 activations +
fp32 outputs) over its own duration, measured with HIP events around each
launch on the launch stream.  Per-shape results for every decode shape, the
prefill product and the decode stack are reported under "shapes".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--quick]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_MFMA_PEAK_TOPS = 5000.0   # MI355X dense int8 matrix-core peak, published
LLC_BYTES = 256 << 20          # Infinity Cache
ROTATE_BYTES = 2 * LLC_BYTES


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--quick", action="store_true", help="headline only (no per-shape table)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


# ----------------------------------------------------------------------------
def gemv_bytes(M, N, K):
    """Algorithmic HBM bytes of one product launch."""
    return N * K // 4 + (N * K // 128) * 4 + M * K + 4 * M + 4 * M * N


class Rotation:
    """R device copies of one packed weight matrix (distinct addresses)."""

    def __init__(self, torch, packed_np, scales_np, min_bytes=ROTATE_BYTES):
        per = packed_np.nbytes + scales_np.nbytes
        self.R = max(2, math.ceil(min_bytes / per))
        p = torch.from_numpy(packed_np).cuda()
        s = torch.from_numpy(scales_np).cuda()
        self.packed = [p] + [p.clone() for _ in range(self.R - 1)]
        self.scales = [s] + [s.clone() for _ in range(self.R - 1)]

    def __getitem__(self, i):
        return self.packed[i % self.R], self.scales[i % self.R]


def time_per_launch(torch, launch, n, stream):
    """Runs launch(i) n times on `stream`, each bracketed by a pair of events.
    Returns (total_ms, per-launch ms array)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(n):
        ev[i][0].record(stream)
        launch(i)
        ev[i][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1), np.array([a.elapsed_time(b) for a, b in ev])


def time_loop(torch, launch, n, stream):
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(n):
        launch(i)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n


# ----------------------------------------------------------------------------
def decode_shape(torch, bn, wl, name, N, K, M, T, S, xbits, iters, warmup, stream):
    """Per-launch timing of quant + product for one decode shape."""
    packed, st = bn.bitnet_pack_i2s(T, S)
    rot = Rotation(torch, packed, st)
    x = torch.from_numpy(xbits.view(np.int16)).cuda().view(torch.bfloat16)
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def step(i):
        bn.bitnet_quant_act(x, q, sa, stream=stream)
        p, s = rot[i]
        bn.bitnet_w2a8_gemv(p, s, q, sa, N, K, y=y, stream=stream)

    def gemv_only(i):
        p, s = rot[i]
        bn.bitnet_w2a8_gemv(p, s, q, sa, N, K, y=y, stream=stream)

    for i in range(warmup):
        step(i)
    step_ms = time_loop(torch, step, iters, stream)
    _, per = time_per_launch(torch, gemv_only, iters, stream)
    loop_ms = time_loop(torch, gemv_only, iters, stream)
    kern_ms = float(np.mean(per))
    pb = N * K // 4
    ab = gemv_bytes(M, N, K)
    return {
        "shape": name, "M": M, "N": N, "K": K, "rotation_copies": rot.R,
        "step_us": step_ms * 1e3,
        "gemv_event_us_mean": kern_ms * 1e3, "gemv_event_us_median": float(np.median(per)) * 1e3,
        "gemv_event_us_min": float(np.min(per)) * 1e3,
        "gemv_loop_us": loop_ms * 1e3,
        "packed_GBps_step": pb / (step_ms * 1e-3) / 1e9,
        "packed_GBps_gemv": pb / (kern_ms * 1e-3) / 1e9,
        "packed_pct_hbm_gemv": 100.0 * pb / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "alg_GBps_gemv": ab / (kern_ms * 1e-3) / 1e9,
        "alg_bytes": ab,
    }


def prefill_shape(torch, bn, wl, iters, warmup, stream):
    c = wl.config4()
    packed, st = bn.bitnet_pack_i2s(c.T, c.S)
    p = torch.from_numpy(packed).cuda()
    s = torch.from_numpy(st).cuda()
    x = torch.from_numpy(c.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    q, sa = bn.bitnet_quant_act(x, stream=stream)
    y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")

    def gemm(i):
        bn.bitnet_w2a8_gemm(p, s, q, sa, c.N, c.K, y=y, stream=stream)

    def step(i):
        bn.bitnet_quant_act(x, q, sa, stream=stream)
        gemm(i)

    for i in range(warmup):
        step(i)
    step_ms = time_loop(torch, step, iters, stream)
    _, per = time_per_launch(torch, gemm, iters, stream)
    kern_ms = float(np.mean(per))
    ops = 2.0 * c.M * c.N * c.K
    return {
        "shape": "gemm_512x13824x2560", "M": c.M, "N": c.N, "K": c.K,
        "step_us": step_ms * 1e3, "gemm_event_us_mean": kern_ms * 1e3,
        "int8_TOPS": ops / (kern_ms * 1e-3) / 1e12,
        "int8_mfma_pct": 100.0 * ops / (kern_ms * 1e-3) / 1e12 / INT8_MFMA_PEAK_TOPS,
    }


# ----------------------------------------------------------------------------
def cpu_baseline(wl, c, T, S, seconds):
    """The oracle, as it stands, timed single-threaded on this host on the
    headline workload (quantise + product of the whole 13824x2560 matrix)."""
    import oracle
    P = oracle.pack_i2s(T)
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    reps = 0
    t0 = time.perf_counter()
    while True:
        q, s = oracle.quant_act_bf16(c.x_bits)
        oracle.w2a8(P, S, q, s, c.N, c.K)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / reps
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": (c.N * c.K // 4) / per / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"{reps} full quantise+product passes of the 13824x2560 M=1 workload "
                  f"({per * 1e3:.1f} ms each, {el:.1f} s), single thread pinned to one core; CPU: {model}",
        "us_per_step": per * 1e6,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
              f"(the product shards by output rows; see the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import bit_gemv_i2_amd as bn
    import workloads as wl

    bn.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---- headline workload: 13824x2560, M=1, absmean-ternarised N(0,0.02) weights
    c = wl.config2(M=1)
    T, S = bn.bitnet_ternarize_absmean(c.W)
    log(f"headline: 13824x2560 M=1, steps={args.steps} warmup={args.warmup}")
    N, K, M = c.N, c.K, c.M
    packed, st = bn.bitnet_pack_i2s(T, S)
    rot = Rotation(torch, packed, st)
    x = torch.from_numpy(c.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    q = torch.empty((M, K), dtype=torch.int8, device=dev)
    sa = torch.empty((M,), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)

    gemv_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]

    def step(i, timed=False):
        bn.bitnet_quant_act(x, q, sa, stream=stream)
        p, s = rot[i]
        if timed:
            gemv_ev[i][0].record(stream)
        bn.bitnet_w2a8_gemv(p, s, q, sa, N, K, y=y, stream=stream)
        if timed:
            gemv_ev[i][1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i, timed=True)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    per = np.array([a.elapsed_time(b) for a, b in gemv_ev])
    kern_ms = float(np.mean(per))
    # a clean pass without the per-launch events, for reference
    clean_ms = time_loop(torch, lambda i: step(i), args.steps, stream)

    pbytes = N * K // 4
    ab = gemv_bytes(M, N, K)
    achieved = ab / (kern_ms * 1e-3) / 1e9
    result = {
        "metric": "W2A8 GEMV packed-weight GB/s, 13824x2560 batch 1 (quant + product per step)",
        "value": pbytes / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8xternary->int32, fp32 epilogue",
        "data": "synthetic (seeded; absmean-ternarised N(0,0.02) weights, N(0,1) bf16 activations)",
        "config": {"workload": "gemv_13824x2560_m1", "M": M, "N": N, "K": K,
                   "rotation_copies": rot.R, "rotation_bytes": rot.R * (packed.nbytes + st.nbytes)},
        "step_us": ms_per_step * 1e3,
        "step_us_without_events": clean_ms * 1e3,
        "pct_hbm_packed": 100.0 * pbytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": {
            "bound": "hbm", "kernel": "gemv_kernel (bitnet_w2a8_gemv)",
            "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": None, "alg_bytes_per_launch": ab,
            "kernel_us_mean": kern_ms * 1e3, "kernel_us_median": float(np.median(per)) * 1e3,
        },
    }
    log(f"headline: {ms_per_step * 1e3:.2f} us/step, gemv {kern_ms * 1e3:.2f} us, "
        f"{result['value']:.0f} GB/s packed per step")

    if not args.quick:
        shapes = []
        iters = max(200, min(2000, args.steps))
        for name, cfg, Ms in [("gemv_2560x2560", 1, [1]), ("gemv_13824x2560", 2, [1, 8]),
                              ("gemv_20480x3200", 3, [1])]:
            for Mi in Ms:
                cc = wl.CONFIGS[cfg](M=Mi)
                if cc.T is None:
                    Tt, Ss = bn.bitnet_ternarize_absmean(cc.W)
                else:
                    Tt, Ss = cc.T, cc.S
                r = decode_shape(torch, bn, wl, name, cc.N, cc.K, Mi, Tt, Ss, cc.x_bits, iters, 50, stream)
                log(json.dumps(r))
                shapes.append(r)
        T5, S5 = wl.stack_matrix(0, 5)
        r = decode_shape(torch, bn, wl, "gemv_2560x6912", 2560, 6912, 1, T5, S5,
                         wl.normal_act(wl.rng_for(5, 99), 1, 6912), iters, 50, stream)
        log(json.dumps(r))
        shapes.append(r)
        r = prefill_shape(torch, bn, wl, 200, 20, stream)
        log(json.dumps(r))
        shapes.append(r)
        result["shapes"] = shapes

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, c, T, S, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
