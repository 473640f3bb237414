#!/usr/bin/env python3
"""Benchmark of the W2A8 ternary decode product on one MI355X.

One step = one pass of the decode hot path over one batch: per-token int8
quantisation of the bf16 activations and the W2A8 product, for the 13824x2560
fused gate+up shape at batch 1 (weights from absmean-ternarised N(0, 0.02),
activations N(0,1) bf16), as one fused launch (bitnet_w2a8_gemv_act, which
quantises exactly as bitnet_quant_act and multiplies as bitnet_w2a8_gemv).
Every step reads a different copy of the packed weights, from a rotation larger
than twice the 256 MB last-level cache, so the weight stream comes from HBM.

value = packed-weight bytes (N*K/4) per step / step time, in GB/s.
The roofline object prices the step's kernel against 8 TB/s using its
algorithmic bytes (packed weights + fp32 block scales + bf16 activations +
fp32 outputs) over its average duration in the timed region (one launch per step;
the steps are timed by HIP events on the launch stream, as the difference of two graph
replays so that the fixed cost of a replay cancels, see config.timing); "product_kernel"
gives the same for the product alone (int8 q in).  Beside them,
"attainable_read" is what one bare pass of 16-byte non-temporal loads (the
hint the product's weight loads carry) over the same number of bytes achieves
on this GPU, and "stream_ceiling_1GiB" what the same read
sustains over 1 GiB; "product_kernel_at_scale" gives the product and the fused
step on a 262144x2560 matrix (189 MB a launch), where per-launch latency no
longer dominates.
Per-shape results for every decode shape, the prefill product, the format
variants, the medium batches and the decode stack are reported under "shapes".
"cpu_baseline" is the CPU oracle, single-threaded, on the headline workload;
"cpu_baseline_all_cores" the same oracle in one process per host core.

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
HEADLINE_PAIRS = 41            # timed replay pairs behind the headline's median (odd)
ROTATE_BYTES = 2 * LLC_BYTES

# HBM bytes per launch of the headline kernels (the fused quantise-and-multiply
# step and the product alone), from two rocprofv3 --pmc passes (FETCH_SIZE,
# WRITE_SIZE) over `bench.py --profile-run`, each scaled by what the counter reads
# for a 64 MiB device copy (FETCH_SIZE x 1.999, WRITE_SIZE x 1.000).  Valid only
# for the kernel source it was taken on.
MEASURED_TRAFFIC = {
    "kernel_source_sha1": "c8f9f93c7838589dd6a845f9c68daf87440c151b",
    "fused": {"bytes_per_launch": 10092703, "fetch_kib": 4903.0, "write_kib": 54.0},
    "product": {"bytes_per_launch": 10076325, "fetch_kib": 4895.0, "write_kib": 54.0},
    "fetch_scale": 1.999, "write_scale": 1.000,
}


def measured_traffic(kernel):
    """The counter-measured bytes of `kernel` ("fused" or "product"), or None if the
    kernel source changed since they were taken."""
    import hashlib
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bit_gemv_i2_amd", "csrc", "bitnet_w2a8.hip")
    try:
        sha = hashlib.sha1(open(path, "rb").read()).hexdigest()
    except OSError:
        return None
    return MEASURED_TRAFFIC[kernel]["bytes_per_launch"] if sha == MEASURED_TRAFFIC["kernel_source_sha1"] else None


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
    ap.add_argument("--profile-stack", action="store_true",
                    help="for a kernel trace: the 30-layer stack's one-token graph (linear fold), replayed 5 times "
                         "at batch 1 and 5 times at batch 8, synchronised after each replay")
    ap.add_argument("--profile-shapes", action="store_true",
                    help="short eager run for counter passes: a 64 MiB device copy (calibration), then 64 product "
                         "launches each of 2560x2560, 2560x6912 and 20480x3200 at batch 1 and 13824x2560 at batch 8")
    ap.add_argument("--profile-run", action="store_true",
                    help="short eager run for hardware-counter passes: a 64 MiB device copy (the byte-count "
                         "calibration), 64 launches each of the headline product and fused step, 16 prefill products")
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


def capture(torch, launch, n):
    """Captures launch(0..n-1) (each enqueuing on the current stream) into one HIP graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(min(n, 4)):
            launch(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            launch(i)
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps, pre=None, warm=True):
    """Replays g `reps` times between two events on the current stream; returns total ms.
    First (untimed) one replay of g when `warm`, a synchronisation, then one replay of
    `pre` (default: g itself) enqueued just before the first event: `pre` covers the whole
    weight rotation, so every timed step finds its weights where the steady state of a
    decode loop leaves them (its copy last read a full rotation, >= 512 MB, earlier, so
    not in the 256 MB last-level cache), and the host submits the timed replays while
    the GPU is still busy with `pre`, so the events bracket the steps' GPU work."""
    stream = torch.cuda.current_stream()
    if warm:
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    (pre or g).replay()
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def steps_by_difference(torch, launch, n, R, reps=10):
    """Times exactly n steady-state steps: graph A runs steps on copies 0..R-1 (one whole
    rotation), graph B the same R steps and then n more on copies 0, 1, ... (so each of the
    n extra steps reads a copy last touched a full rotation earlier, as in a decode loop).
    Each replay is timed by events on the launch stream, behind an untimed full rotation
    that hides the host's submission.  T(B) - T(A) holds exactly the n extra steps' GPU
    work: the fixed cost of a graph replay (the same in both) cancels.  Returns the
    per-repeat differences in ms (A and B alternate, `reps` times)."""
    gA = capture(torch, launch, R)
    gB = capture(torch, lambda i: launch(i if i < R else i - R), R + n)
    gA.replay()
    gB.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        a = time_graph(torch, gA, 1, pre=gA, warm=False)
        b = time_graph(torch, gB, 1, pre=gA, warm=False)
        out.append(b - a)
    del gA, gB
    return out


def graph_us_per_launch(torch, launch, n, reps):
    g = capture(torch, launch, n)
    return time_graph(torch, g, reps) * 1e3 / (n * reps)


def eager_us_per_launch(torch, launch, n):
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(n):
        launch(i)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / n


# ----------------------------------------------------------------------------
class DecodeShape:
    """Device buffers of one decode workload: a rotation of packed weights,
    bf16 activations, int8/scale scratch and fp32 outputs."""

    def __init__(self, torch, bn, name, N, K, M, T, S, xbits):
        self.torch, self.bn, self.name, self.N, self.K, self.M = torch, bn, name, N, K, M
        packed, st = bn.bitnet_pack_i2s(T, S)
        self.rot = Rotation(torch, packed, st)
        self.packed_bytes = packed.nbytes
        self.x = torch.from_numpy(xbits.view(np.int16)).cuda().view(torch.bfloat16)
        self.q = torch.empty((M, K), dtype=torch.int8, device="cuda")
        self.sa = torch.empty((M,), dtype=torch.float32, device="cuda")
        self.y = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def quant(self, i):
        self.bn.bitnet_quant_act(self.x, self.q, self.sa)

    def gemv(self, i):
        p, s = self.rot[i]
        self.bn.bitnet_w2a8_gemv(p, s, self.q, self.sa, self.N, self.K, y=self.y)

    def step2(self, i):
        """Two launches: quantise, then multiply."""
        self.quant(i)
        self.gemv(i)

    def fused(self, i):
        """One launch: quantise-and-multiply."""
        p, s = self.rot[i]
        self.bn.bitnet_w2a8_gemv_act(p, s, self.x, self.N, self.K, y=self.y)

    def measure(self, reps=20):
        torch = self.torch
        n = self.rot.R
        step2_us = graph_us_per_launch(torch, self.step2, n, reps)
        fused_us = graph_us_per_launch(torch, self.fused, n, reps)
        gemv_us = graph_us_per_launch(torch, self.gemv, n, reps)
        quant_us = graph_us_per_launch(torch, self.quant, 64, reps)
        pb = self.packed_bytes
        ab = gemv_bytes(self.M, self.N, self.K)
        best = min(step2_us, fused_us)
        return {
            "shape": self.name, "M": self.M, "N": self.N, "K": self.K, "rotation_copies": n,
            "step_us": best, "step_two_launch_us": step2_us, "step_fused_us": fused_us,
            "gemv_us": gemv_us, "quant_us": quant_us,
            "packed_GBps_step": pb / best / 1e3, "packed_GBps_gemv": pb / gemv_us / 1e3,
            "packed_pct_hbm_gemv": 100.0 * pb / gemv_us / 1e3 / HBM_PEAK_GBS,
            "alg_GBps_gemv": ab / gemv_us / 1e3, "alg_bytes": ab,
        }


def attainable_read(torch, bn, nbytes, reps=10):
    """Graph-timed plain stream read (bitnet_probe_stream_read) of nbytes, rounded
    up to 16, cycling through copies larger than twice the last-level cache: what
    a bare one-pass read of the product kernel's bytes attains on this GPU."""
    n = (nbytes + 15) // 16 * 16
    nrot = max(2, math.ceil(ROTATE_BYTES / n))
    bufs = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(nrot)]
    sink = torch.empty((bn.lib().bitnet_probe_stream_read_sink_len(n),), dtype=torch.int32, device="cuda")
    us = graph_us_per_launch(torch, lambda i: bn.bitnet_probe_stream_read(bufs[i % nrot], sink, 0), nrot, reps)
    us_noout = graph_us_per_launch(torch, lambda i: bn.bitnet_probe_stream_read(bufs[i % nrot], sink, 1), nrot, reps)
    del bufs
    torch.cuda.empty_cache()
    return {"what": "one pass of 16-byte non-temporal loads, one per thread, over the same number of bytes, each wave storing "
                    "one word (bitnet_probe_stream_read mode 0); no_output: the same read storing nothing (mode 1)",
            "bytes": n, "us": us, "GBps": n / us / 1e3, "no_output_us": us_noout, "no_output_GBps": n / us_noout / 1e3}


def stream_ceiling(torch, bn, reps=5):
    """Graph-timed one-pass read of 1 GiB (bitnet_probe_stream_read, two buffers
    alternating, each four times the last-level cache): the streaming-read rate
    this GPU sustains when launch and ramp costs are amortised."""
    n = 1 << 30
    bufs = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(2)]
    sink = torch.empty((bn.lib().bitnet_probe_stream_read_sink_len(n),), dtype=torch.int32, device="cuda")
    us = graph_us_per_launch(torch, lambda i: bn.bitnet_probe_stream_read(bufs[i % 2], sink, 0), 2, reps)
    del bufs, sink
    torch.cuda.empty_cache()
    return {"what": "one-pass read of 1 GiB, 16-byte non-temporal loads (bitnet_probe_stream_read mode 0)",
            "bytes": n, "us": us, "GBps": n / us / 1e3}


def product_at_scale(torch, bn, wl, N=262144, K=2560, reps=5):
    """The decode product and the fused step at batch 1 on a tall matrix (262144 x 2560,
    189 MB a launch, iid uniform ternary weights, rotated past the last-level cache): the
    kernel's streaming rate once per-launch latency is amortised over a large stream."""
    r = wl.rng_for(7, N, K)
    packed, st = bn.bitnet_pack_i2s(wl.ternary_uniform(r, N, K), wl.uniform_scales(r, N, K))
    rot = Rotation(torch, packed, st)
    del packed, st
    xb = wl.normal_act(wl.rng_for(8, K), 1, K)
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    q, sa = bn.bitnet_quant_act(x)
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")

    def gemv(i):
        p, s = rot[i]
        bn.bitnet_w2a8_gemv(p, s, q, sa, N, K, y=y)

    def fused(i):
        p, s = rot[i]
        bn.bitnet_w2a8_gemv_act(p, s, x, N, K, y=y)

    n = max(rot.R, 4)
    gemv_us = graph_us_per_launch(torch, gemv, n, reps)
    fused_us = graph_us_per_launch(torch, fused, n, reps)
    ab = gemv_bytes(1, N, K)
    out = {"kernel": "gemv_kernel (bitnet_w2a8_gemv, int8 q in) and the fused step (bitnet_w2a8_gemv_act), "
                     f"{N}x{K} batch 1, graph-timed over {rot.R} weight copies",
           "N": N, "K": K, "M": 1, "alg_bytes_per_launch": ab, "kernel_us": gemv_us,
           "achieved": ab / gemv_us / 1e3, "frac": ab / gemv_us / 1e3 / HBM_PEAK_GBS,
           "fused_kernel_us": fused_us, "fused_achieved": (ab + K) / fused_us / 1e3,
           "fused_frac": (ab + K) / fused_us / 1e3 / HBM_PEAK_GBS}
    del rot
    torch.cuda.empty_cache()
    return out


def prefill_shape(torch, bn, wl, reps=10):
    c = wl.config4()
    packed, st = bn.bitnet_pack_i2s(c.T, c.S)
    p = torch.from_numpy(packed).cuda()
    s = torch.from_numpy(st).cuda()
    x = torch.from_numpy(c.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    q, sa = bn.bitnet_quant_act(x)
    y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")

    def gemm(i):
        bn.bitnet_w2a8_gemm(p, s, q, sa, c.N, c.K, y=y)

    def step(i):
        bn.bitnet_quant_act(x, q, sa)
        gemm(i)

    gemm_us = graph_us_per_launch(torch, gemm, 20, reps)
    step_us = graph_us_per_launch(torch, step, 20, reps)
    ops = 2.0 * c.M * c.N * c.K
    return {
        "shape": "gemm_512x13824x2560", "M": c.M, "N": c.N, "K": c.K,
        "step_us": step_us, "gemm_us": gemm_us,
        "int8_TOPS": ops / gemm_us / 1e6,
        "int8_mfma_pct": 100.0 * ops / gemm_us / 1e6 / INT8_MFMA_PEAK_TOPS,
    }


def stack_shape(torch, bn, wl, runs=((1, "sum"), (8, "sum"), (1, "relu2_glu")), reps=20):
    """The 30-layer decode stack (4 x 2560x2560, 13824x2560, 2560x6912 per layer):
    one token = one bitnet_w2a8_chain call (180 products), captured as a graph.
    The junction in front of each 2560x6912 layer is the linear fold (the
    headline stack) or the squared-ReLU gate."""
    t0 = time.perf_counter()
    ws, pbytes = [], 0
    for layer in range(wl.STACK_LAYERS):
        for idx in range(6):
            T, S = wl.stack_matrix(layer, idx)
            ws.append(bn.PackedWeight.from_ternary(T, S))
            pbytes += T.size // 4
    setup_s = time.perf_counter() - t0
    out = []
    for M, junction in runs:
        chain = bn.Chain(ws, [junction if i % 6 == 5 else False for i in range(len(ws))])
        x = torch.from_numpy(wl.stack_input(M).view(np.int16)).cuda().view(torch.bfloat16)
        y = torch.empty((M, wl.STACK_HIDDEN), dtype=torch.float32, device="cuda")
        chain.workspace(M)
        us = graph_us_per_launch(torch, lambda i: chain(x, y=y), 1, reps)
        row = {"shape": "stack_30x6_decode", "M": M, "junction": junction, "token_step_us": us,
               "tokens_per_s": M * 1e6 / us, "products_per_token": len(ws), "packed_bytes_per_token": pbytes,
               "packed_GBps": pbytes / us / 1e3, "pct_hbm_packed": 100.0 * pbytes / us / 1e3 / HBM_PEAK_GBS,
               "setup_s": setup_s}
        if M == 1:  # the one-launch persistent form of the same token (plan and workspace made eagerly first)
            chain.persistent(x, y=y)
            torch.cuda.synchronize()
            pus = graph_us_per_launch(torch, lambda i: chain.persistent(x, y=y), 1, reps)
            torch.cuda.synchronize()
            row["persistent_token_step_us"] = pus
            row["persistent_status"] = chain.persistent_layer_outputs(1, bn.BITNET_DT_BF16)[1]
        out.append(row)
        del chain
    del ws
    torch.cuda.empty_cache()
    return out


def format_shapes(torch, bn, wl, reps=10):
    """Scale-granularity variants (64-weight blocks, one scale per matrix) of the
    13824x2560 decode product (M=1, rotated weights) and the 512-token prefill."""
    c = wl.config4()
    x = torch.from_numpy(c.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    q, sa = bn.bitnet_quant_act(x)
    q1, sa1 = q[:1].contiguous(), sa[:1].contiguous()
    r = wl.rng_for(4, 7)
    out = []
    for G in (64, 0):
        S = r.uniform(0.5, 2, size=(1,) if G == 0 else (c.N, c.K // G)).astype(np.float32)
        packed, st = bn.bitnet_pack_i2s_g(c.T, S, G)
        nrot = max(2, math.ceil(ROTATE_BYTES / (packed.nbytes + st.nbytes)))
        P = [torch.from_numpy(packed).cuda() for _ in range(nrot)]
        Sd = [torch.from_numpy(st).cuda() for _ in range(nrot)]
        y1 = torch.empty((1, c.N), dtype=torch.float32, device="cuda")
        gemv_us = graph_us_per_launch(torch, lambda i: bn.bitnet_w2a8_gemv_g(P[i % nrot], Sd[i % nrot], q1, sa1, c.N,
                                                                              c.K, G, y=y1), nrot, reps)
        yb = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
        gemm_us = graph_us_per_launch(torch, lambda i: bn.bitnet_w2a8_gemm_g(P[0], Sd[0], q, sa, c.N, c.K, G, y=yb),
                                      20, reps)
        ops = 2.0 * c.M * c.N * c.K
        out.append({"shape": "formats_13824x2560", "scale_block": G, "gemv_m1_us": gemv_us,
                    "gemv_packed_GBps": c.N * c.K / 4 / gemv_us / 1e3, "gemm_m512_us": gemm_us,
                    "gemm_int8_mfma_pct": 100.0 * ops / gemm_us / 1e6 / INT8_MFMA_PEAK_TOPS})
        del P, Sd
        torch.cuda.empty_cache()
    return out


def lut_shapes(torch, bn, wl, reps=10, tiles=(1, 2, 4)):
    """The table-lookup decode product (bitnet_w2a8_gemv_lut, one token) beside the
    matrix-core product on the same weight rotation, for the four decode shapes."""
    out = []
    cases = [("2560x2560", 1), ("13824x2560", 2), ("20480x3200", 3), ("2560x6912", None)]
    for name, cfg in cases:
        if cfg is None:
            T, S = wl.stack_matrix(0, 5)
            N, K = T.shape
            xbits = wl.normal_act(wl.rng_for(5, 99), 1, K)
        else:
            cc = wl.CONFIGS[cfg](M=1)
            T, S = (bn.bitnet_ternarize_absmean(cc.W) if cc.T is None else (cc.T, cc.S))
            N, K, xbits = cc.N, cc.K, cc.x_bits
        ds = DecodeShape(torch, bn, "lut_" + name, N, K, 1, T, S, xbits)
        ds.quant(0)
        n = ds.rot.R
        r = {"shape": "lut_gemv_" + name, "M": 1, "N": N, "K": K, "rotation_copies": n,
             "mfma_gemv_us": graph_us_per_launch(torch, ds.gemv, n, reps)}
        for t in tiles:
            def lut(i, t=t):
                p, s = ds.rot[i]
                bn.bitnet_w2a8_gemv_lut(p, s, ds.q, ds.sa, N, K, t, y=ds.y)
            us = graph_us_per_launch(torch, lut, n, reps)
            r[f"lut_us_tiles{t}"] = us
            r[f"lut_packed_GBps_tiles{t}"] = N * K / 4 / us / 1e3
        r["lut_over_mfma_best"] = min(r[f"lut_us_tiles{t}"] for t in tiles) / r["mfma_gemv_us"]
        del ds
        torch.cuda.empty_cache()
        out.append(r)
    return out


def medium_batch_shapes(torch, bn, wl, reps=10):
    """13824x2560 between decode and prefill: the decode kernel up to M=16, the
    prefill kernel from M=16 to 128 (weights rotated through HBM for both)."""
    c = wl.config4()
    x = torch.from_numpy(c.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    q, sa = bn.bitnet_quant_act(x)
    rot = Rotation(torch, *bn.bitnet_pack_i2s(c.T, c.S))
    pbytes = c.N * c.K // 4
    out = []
    for M in (16, 32, 64, 128):
        qm, sm = q[:M].contiguous(), sa[:M].contiguous()
        row = {"shape": "medium_batch_13824x2560", "M": M}
        if M <= 16:
            y = torch.empty((M, c.N), dtype=torch.float32, device="cuda")
            us = graph_us_per_launch(torch, lambda i: bn.bitnet_w2a8_gemv(*rot[i], qm, sm, c.N, c.K, y=y), rot.R, reps)
            row.update({"gemv_us": us, "gemv_packed_GBps": pbytes / us / 1e3})
        yb = torch.empty((M, c.N), dtype=torch.bfloat16, device="cuda")
        us = graph_us_per_launch(torch, lambda i: bn.bitnet_w2a8_gemm(*rot[i], qm, sm, c.N, c.K, y=yb), rot.R, reps)
        row.update({"gemm_us": us, "gemm_packed_GBps": pbytes / us / 1e3,
                    "gemm_int8_TOPS": 2.0 * M * c.N * c.K / us / 1e6})
        out.append(row)
    del rot
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
def _oracle_passes(args):
    """One host core: the oracle's quantise + product passes on the headline
    workload for about `seconds` (runs in a process of its own)."""
    core, P, S, x_bits, N, K, seconds = args
    try:
        os.sched_setaffinity(0, {core})
    except (AttributeError, OSError):
        pass
    import oracle
    reps, t0 = 0, time.perf_counter()
    while True:
        q, s = oracle.quant_act_bf16(x_bits)
        oracle.w2a8(P, S, q, s, N, K)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return reps, el


def cpu_baseline_all_cores(c, T, S, seconds, cores):
    """The same oracle on every host core this process may use (at most 16): one
    process per core, each running independent single-threaded passes; the
    aggregate rate of all of them."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    import oracle
    P = oracle.pack_i2s(T)
    use = list(cores)[:16]
    # fresh interpreters that never touch the GPU; a worker that fails raises here
    with ProcessPoolExecutor(max_workers=len(use), mp_context=mp.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_passes, [(k, P, S, c.x_bits, c.N, c.K, seconds) for k in use],
                          timeout=seconds + 120))
    reps = sum(r for r, _ in res)
    wall = max(e for _, e in res)
    return {
        "value": reps * (c.N * c.K // 4) / wall / 1e9, "unit": "GB/s", "cores": len(use), "kind": "oracle",
        "sample": f"{reps} full quantise+product passes of the 13824x2560 M=1 workload in {len(use)} "
                  f"processes, one pinned to each core, {wall:.1f} s",
    }


def cpu_baseline(wl, c, T, S, seconds, y_gpu=None):
    """The oracle, as it stands, timed single-threaded on this host on the
    headline workload (quantise + product of the whole 13824x2560 matrix).  Its
    result is also compared with the GPU's headline output: the worst error as a
    fraction of the tolerance 1e-5 * max(|y|, mag) and the plain maximum relative
    error."""
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
    parity = None
    if y_gpu is not None:
        ref = oracle.w2a8(P, S, q, s, c.N, c.K)
        err = np.abs(y_gpu.astype(np.float64) - ref["y64"])
        bound = 1e-5 * np.maximum(np.abs(ref["y64"]), ref["mag"])
        nz = ref["y64"] != 0
        parity = {"outputs": int(err.size), "worst_err_over_tolerance": float((err / bound).max()),
                  "outside_tolerance": int(np.count_nonzero(err > bound)),
                  "plain_max_rel_err": float((err[nz] / np.abs(ref["y64"][nz])).max())}
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
        "parity_of_gpu_headline_output": parity,
    }


def profile_run(torch, bn, wl):
    """Known-size copy first (counter calibration), then the headline kernels."""
    n = 64 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    c = wl.config2(M=1)
    T, S = bn.bitnet_ternarize_absmean(c.W)
    d = DecodeShape(torch, bn, "gemv_13824x2560", c.N, c.K, c.M, T, S, c.x_bits)
    d.quant(0)
    torch.cuda.synchronize()
    for i in range(64):
        d.gemv(i)
    torch.cuda.synchronize()
    for i in range(64):
        d.fused(i)
    torch.cuda.synchronize()
    for i in range(64):
        p, s = d.rot[i]
        bn.bitnet_w2a8_gemv_lut(p, s, d.q, d.sa, c.N, c.K, 2, y=d.y)
    torch.cuda.synchronize()
    del d
    c4 = wl.config4()
    w4 = bn.PackedWeight.from_ternary(c4.T, c4.S)
    x4 = torch.from_numpy(c4.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    q4, s4 = bn.bitnet_quant_act(x4)
    y4 = torch.empty((c4.M, c4.N), dtype=torch.bfloat16, device="cuda")
    for i in range(16):
        w4.gemm(q4, s4, y=y4)
    torch.cuda.synchronize()
    log(f"profile run done: copy {n} B x3, gemv x64, fused x64, lut gemv x64, prefill 512x13824x2560 x16")


def calibration_copy(torch):
    """A plain 64 MiB device copy, three times: the known byte count the HBM counters are scaled by."""
    n = 64 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def profile_stack(torch, bn, wl):
    """One token of the 30-layer stack (180 products, linear fold) captured as a graph,
    replayed 5 times at batch 1 and 5 times at batch 8, with a synchronisation after
    every replay so each token stands alone in the trace; at batch 1 also the same token
    as one persistent launch (bitnet_w2a8_chain_persistent), replayed 5 times."""
    ws = []
    for layer in range(wl.STACK_LAYERS):
        for idx in range(6):
            T, S = wl.stack_matrix(layer, idx)
            ws.append(bn.PackedWeight.from_ternary(T, S))
    for M in (1, 8):
        chain = bn.Chain(ws, ["sum" if i % 6 == 5 else False for i in range(len(ws))])
        x = torch.from_numpy(wl.stack_input(M).view(np.int16)).cuda().view(torch.bfloat16)
        y = torch.empty((M, wl.STACK_HIDDEN), dtype=torch.float32, device="cuda")
        chain.workspace(M)
        g = capture(torch, lambda i: chain(x, y=y), 1)
        for _ in range(5):
            g.replay()
            torch.cuda.synchronize()
        log(f"profile stack: batch {M}, 5 token replays done")
        del g
        if M == 1:  # the same token as one persistent launch (after its fill launch)
            chain.persistent(x, y=y)
            torch.cuda.synchronize()
            g = capture(torch, lambda i: chain.persistent(x, y=y), 1)
            for _ in range(5):
                g.replay()
                torch.cuda.synchronize()
            status = chain.persistent_layer_outputs(1, bn.BITNET_DT_BF16)[1]
            log(f"profile stack: batch 1 persistent, 5 token replays done (status {status})")
            del g
        del chain


def profile_shapes(torch, bn, wl):
    """Counter passes over the decode shapes besides the headline: 64 product launches
    each (weights rotated past the last-level cache) of 2560x2560, 2560x6912 and
    20480x3200 at batch 1 and of 13824x2560 at batch 8."""
    calibration_copy(torch)
    cases = []
    c1 = wl.config1()
    cases.append(("gemv_2560x2560", c1.N, c1.K, 1, c1.T, c1.S, c1.x_bits))
    T5, S5 = wl.stack_matrix(0, 5)
    cases.append(("gemv_2560x6912", 2560, 6912, 1, T5, S5, wl.normal_act(wl.rng_for(5, 99), 1, 6912)))
    c3 = wl.config3()
    cases.append(("gemv_20480x3200", c3.N, c3.K, 1, c3.T, c3.S, c3.x_bits))
    c2 = wl.config2(M=8)
    T2, S2 = bn.bitnet_ternarize_absmean(c2.W)
    cases.append(("gemv_13824x2560_m8", c2.N, c2.K, 8, T2, S2, c2.x_bits))
    for name, N, K, M, T, S, xb in cases:
        d = DecodeShape(torch, bn, name, N, K, M, T, S, xb)
        d.quant(0)
        torch.cuda.synchronize()
        for i in range(64):
            d.gemv(i)
        torch.cuda.synchronize()
        log(f"profile shapes: {name} batch {M}: 64 product launches done")
        del d
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the product would shard by output rows; see the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import bit_gemv_i2_amd as bn
    import workloads as wl

    bn.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    if args.profile_run:
        profile_run(torch, bn, wl)
        return
    if args.profile_stack:
        profile_stack(torch, bn, wl)
        return
    if args.profile_shapes:
        profile_shapes(torch, bn, wl)
        return

    # ---- headline workload: 13824x2560, M=1, absmean-ternarised N(0,0.02) weights
    c = wl.config2(M=1)
    T, S = bn.bitnet_ternarize_absmean(c.W)
    log(f"headline: 13824x2560 M=1, steps={args.steps} warmup={args.warmup}")
    d = DecodeShape(torch, bn, "gemv_13824x2560", c.N, c.K, c.M, T, S, c.x_bits)
    for i in range(args.warmup):
        d.fused(i)
    torch.cuda.synchronize()
    # exactly `steps` decode steps (one quantise-and-multiply launch each, step i on
    # weight copy i mod R); for reference also timed as one replay of a graph of just them
    g = capture(torch, d.fused, args.steps)
    g_rot = capture(torch, d.fused, d.rot.R)
    whole_replay_ms = time_graph(torch, g, 1, pre=g_rot)
    # `steps` steady-state steps, as the difference of two event-timed graph replays (one
    # rotation, and the same rotation followed by the `steps` steps): the median of 41 pairs
    diffs = sorted(steps_by_difference(torch, d.fused, args.steps, d.rot.R, reps=HEADLINE_PAIRS))
    total_ms = diffs[HEADLINE_PAIRS // 2]
    ms_per_step = total_ms / args.steps
    # what one replay of a graph of just the `steps` steps costs beyond them (not in `value`)
    graph_replay_fixed_us = (whole_replay_ms - total_ms) * 1e3
    # the product kernel alone (pre-quantised input): one graph over the weight rotation
    reps = max(1, args.steps // d.rot.R)
    gemv_us = graph_us_per_launch(torch, d.gemv, d.rot.R, reps)
    quant_us = graph_us_per_launch(torch, d.quant, 64, 10)
    step2_us = graph_us_per_launch(torch, d.step2, d.rot.R, reps)
    eager_us = eager_us_per_launch(torch, d.fused, min(args.steps, 500))
    # spread over the timed pairs (the median is `value`)
    rep_us = [x * 1e3 / args.steps for x in diffs]
    del g, g_rot
    y_headline = d.y.cpu().numpy().copy()

    N, K, M = c.N, c.K, c.M
    pbytes = N * K // 4
    ab = gemv_bytes(M, N, K)
    ab_fused = ab + M * K  # bf16 activations (2 bytes a value) instead of int8 q
    step_us = ms_per_step * 1e3  # one fused launch per step: its average duration over the timed region
    achieved = ab_fused / step_us / 1e3
    achieved_product = ab / gemv_us / 1e3
    attain = attainable_read(torch, bn, ab_fused, reps)
    attain["fused_frac_of_attainable"] = achieved / attain["GBps"]
    attain["product_frac_of_attainable"] = achieved_product / attain["GBps"]
    ceiling = stream_ceiling(torch, bn)
    ceiling["fused_frac_of_ceiling"] = achieved / ceiling["GBps"]
    at_scale = product_at_scale(torch, bn, wl)
    at_scale["frac_of_stream_ceiling"] = at_scale["achieved"] / ceiling["GBps"]
    result = {
        "metric": "W2A8 GEMV packed-weight GB/s, 13824x2560 batch 1 (quantise + product per step)",
        "value": pbytes / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "arithmetic": "int8 activations x ternary weights -> int32 per 128-weight block, fp32 epilogue",
        "data": "synthetic (seeded; absmean-ternarised N(0,0.02) weights, N(0,1) bf16 activations)",
        "config": {"workload": "gemv_13824x2560_m1", "M": M, "N": N, "K": K,
                   "rotation_copies": d.rot.R, "rotation_bytes": d.rot.R * (pbytes + N * K // 32),
                   "timed_copies": min(args.steps, d.rot.R),
                   "timed_weight_bytes": args.steps * (pbytes + N * K // 32),
                   "timing": "exactly `steps` steps, step i on weight copy i mod rotation_copies, in the "
                             "steady state of the rotation (rotation_bytes >= 2 x the 256 MB last-level cache: "
                             "each step reads a copy last touched a full rotation earlier); timed as the "
                             "difference of two event-timed replays of HIP graphs, one over a whole rotation "
                             "and one over the same rotation followed by the `steps` steps, so the fixed cost "
                             "of a graph replay cancels (median of 41 pairs); step_us_whole_replay times one "
                             "replay of a graph of just the `steps` steps instead, that fixed cost "
                             "(graph_replay_fixed_us) included"},
        "graph_replay_fixed_us": graph_replay_fixed_us,
        "step_us_whole_replay": whole_replay_ms * 1e3 / args.steps,
        "step_us": ms_per_step * 1e3,
        "step_us_repeats": {"n": len(rep_us), "median": rep_us[len(rep_us) // 2], "min": rep_us[0],
                            "max": rep_us[-1]},
        "pct_hbm_packed_step": 100.0 * pbytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "quant_us": quant_us,
        "step_two_launch_us": step2_us,
        "eager_step_us": eager_us,
        "roofline": {
            "bound": "hbm",
            "kernel": "gemv_kernel, fused quantise-and-multiply form (bitnet_w2a8_gemv_act): the step's one launch",
            "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic("fused"), "alg_bytes_per_launch": ab_fused, "kernel_us": step_us,
            "attainable_read": attain,
            "stream_ceiling_1GiB": ceiling,
            "product_kernel": {
                "kernel": "gemv_kernel (bitnet_w2a8_gemv, int8 q in), graph-timed over the weight rotation",
                "achieved": achieved_product, "frac": achieved_product / HBM_PEAK_GBS, "kernel_us": gemv_us,
                "alg_bytes_per_launch": ab, "traffic": measured_traffic("product"),
                "packed_GBps_kernel": pbytes / gemv_us / 1e3,
            },
            "product_kernel_at_scale": at_scale,
        },
    }
    log(f"headline: a replay of a graph of just the {args.steps} steps takes {whole_replay_ms * 1e3:.1f} us "
        f"({whole_replay_ms * 1e3 / args.steps:.2f} us a step): {graph_replay_fixed_us:.1f} us of fixed cost per "
        f"graph replay on the GPU (not in the timed steps)")
    log(f"headline: {ms_per_step * 1e3:.2f} us/step ({result['value']:.0f} GB/s packed), "
        f"gemv {gemv_us:.2f} us, quant {quant_us:.2f} us, two-launch step {step2_us:.2f} us, "
        f"eager step {eager_us:.2f} us; a bare read of the same {attain['bytes']} B takes {attain['us']:.2f} us "
        f"({attain['GBps']:.0f} GB/s); "
        f"a 1 GiB read streams at {ceiling['GBps']:.0f} GB/s")
    del d
    torch.cuda.empty_cache()

    if not args.quick:
        shapes = []
        for name, cfg, Ms in [("gemv_2560x2560", 1, [1]), ("gemv_13824x2560", 2, [1, 8]),
                              ("gemv_20480x3200", 3, [1])]:
            for Mi in Ms:
                cc = wl.CONFIGS[cfg](M=Mi)
                if cc.T is None:
                    Tt, Ss = bn.bitnet_ternarize_absmean(cc.W)
                else:
                    Tt, Ss = cc.T, cc.S
                ds = DecodeShape(torch, bn, name, cc.N, cc.K, Mi, Tt, Ss, cc.x_bits)
                r = ds.measure()
                del ds
                torch.cuda.empty_cache()
                log(json.dumps(r))
                shapes.append(r)
        T5, S5 = wl.stack_matrix(0, 5)
        ds = DecodeShape(torch, bn, "gemv_2560x6912", 2560, 6912, 1, T5, S5,
                         wl.normal_act(wl.rng_for(5, 99), 1, 6912))
        r = ds.measure()
        del ds
        log(json.dumps(r))
        shapes.append(r)
        r = prefill_shape(torch, bn, wl)
        log(json.dumps(r))
        shapes.append(r)
        for r in format_shapes(torch, bn, wl) + medium_batch_shapes(torch, bn, wl) + lut_shapes(torch, bn, wl):
            log(json.dumps(r))
            shapes.append(r)
        for r in stack_shape(torch, bn, wl):
            log(json.dumps(r))
            shapes.append(r)
        result["shapes"] = shapes

    if not args.no_cpu:
        cores = sorted(os.sched_getaffinity(0))
        result["cpu_baseline_all_cores"] = cpu_baseline_all_cores(c, T, S, min(args.cpu_seconds, 8.0), cores)
        result["cpu_baseline"] = cpu_baseline(wl, c, T, S, args.cpu_seconds, y_headline)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
