"""Process pool that runs the CPU oracle for the full-size GPU parity tests.

Test infrastructure.  The workers are fresh interpreters (spawn) that import
only numpy, the oracle and the seeded input generators -- never torch or the
HIP library -- regenerate the seeded weights they need from those generators,
and return what the oracle finds for the GPU results they are handed.  Splitting
the work by output rows or by product changes no result: rows and products
are independent in the oracle's definition.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

RTOL = 1e-5


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pool() -> ProcessPoolExecutor:
    return ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"))


def f32_check(y, y64, mag):
    """Worst error / bound ratio, count outside 1e-5 * max(|y|, mag), and the plain
    maximum relative error |y - y64| / |y64| over the nonzero exact values."""
    bound = RTOL * np.maximum(np.abs(y64), mag)
    err = np.abs(y.astype(np.float64) - y64)
    nz = y64 != 0
    plain = float((err[nz] / np.abs(y64[nz])).max()) if nz.any() else 0.0
    ratio = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    return ratio, int(np.count_nonzero(err > bound)), plain


# ------------------------------------------------------------------ prefill, 512 x 13824 x 2560
def config4_rows(n0: int, n1: int):
    """The oracle's int32 sums, exact values and magnitudes of rows [n0, n1) of the
    512 x 13824 x 2560 prefill workload, for every token."""
    import oracle
    import workloads as wl
    c = wl.config4()
    q, s = oracle.quant_act_bf16(c.x_bits)
    r = oracle.w2a8(oracle.pack_i2s(c.T[n0:n1]), c.S[n0:n1], q, s, n1 - n0, c.K)
    return n0, r["acc"], r["y64"], r["mag"]


# ------------------------------------------------------------------ the decode stack
def quantise(kind: str, h):
    """The oracle's quantisation of a layer input: "bf16" bit patterns, "plain" fp32,
    or the junctions "sum" / "relu2_glu" of a two-half fp32 output."""
    import oracle
    if kind == "bf16":
        return oracle.quant_act_bf16(h)
    if kind == "plain":
        return oracle.quant_act_f32(h)
    if kind == "sum":
        return oracle.fold_quant(h)
    if kind == "relu2_glu":
        return oracle.glu_quant(h)
    raise ValueError(kind)


def exact_input(kind: str, y64, mag):
    """The exact (fp64) quantiser input a layer would see from the exact outputs y64 of
    the layer before, and a bound on how far any evaluation within the product
    tolerance (|y - y64| <= 1e-5 max(|y64|, mag)) can move it, before fp32 rounding."""
    tau = RTOL * np.maximum(np.abs(y64), mag)
    if kind == "plain":
        return y64, tau
    H = y64.shape[1] // 2
    lo, hi, tl, th = y64[:, :H], y64[:, H:], tau[:, :H], tau[:, H:]
    if kind == "sum":
        return lo + hi, tl + th
    if kind == "relu2_glu":
        g = np.maximum(lo, 0.0)
        # d(g^2 u) = 2 g u dg + g^2 du (+ the second-order terms, bounded by doubling)
        return g * g * hi, 2.0 * (2.0 * g * np.abs(hi) * tl + g * g * th + tl * tl * np.abs(hi))
    raise ValueError(kind)


def decision_check(kind: str, y_gpu, y_own, y64, mag):
    """R11 with identical inputs: the GPU's fp32 outputs and the oracle's own fp32
    outputs of the same product (same input codes) are both quantised for the next
    layer by the oracle's quantiser.  Codes may differ only where the exact input
    lies within the error band of a rounding midpoint, and then by exactly one.
    Returns (number of differing codes, max |dq|, number of differing codes NOT at
    a midpoint, number of codes)."""
    qg, _ = quantise(kind, y_gpu)
    qo, _ = quantise(kind, y_own)
    diff = qg != qo
    n = int(np.count_nonzero(diff))
    if n == 0:
        return 0, 0, 0, int(qg.size)
    dq = int(np.abs(qg.astype(np.int32) - qo.astype(np.int32)).max())
    h64, tau_h = exact_input(kind, y64, mag)
    amax = np.maximum(np.abs(h64).max(axis=1, keepdims=True), 1e-5)
    tau_amax = tau_h.max(axis=1, keepdims=True)
    inv = 127.0 / amax
    v = h64 * inv
    band = 2.0 * (inv * tau_h + np.abs(v) * tau_amax / amax) + np.abs(v) * 2.0 ** -20 + 2.0 ** -30
    dist = np.abs(np.abs(v - np.floor(v)) - 0.5)  # distance to the nearest half-integer
    unjustified = int(np.count_nonzero(diff & (dist > band)))
    return n, dq, unjustified, int(qg.size)


def stack_product(task):
    """One product of the decode stack, layer-local: the oracle is fed the GPU's own
    input to this product (its previous fp32 output, or the bf16 token) for every
    batch size, and compares the GPU's output element by element; then it checks the
    requantisation decisions of the next junction (R11 with identical inputs).

    task = (p, layer, idx, kind, next_kind, runs) with runs = [(M, input, y_gpu), ...]."""
    import oracle
    import workloads as wl
    p, layer, idx, kind, next_kind, runs = task
    T, S = wl.stack_matrix(layer, idx)
    N, K = T.shape
    P = oracle.pack_i2s(T)
    out = []
    for M, inp, y_gpu in runs:
        q, s = quantise(kind, inp)
        r = oracle.w2a8(P, S, q, s, N, K)
        ratio, bad, plain = f32_check(y_gpu, r["y64"], r["mag"])
        dec = decision_check(next_kind, y_gpu, r["y"], r["y64"], r["mag"]) if next_kind else (0, 0, 0, 0)
        out.append({"p": p, "M": M, "ratio": ratio, "bad": bad, "plain_rel": plain, "n_diff": dec[0],
                    "max_dq": dec[1], "unjustified": dec[2], "codes": dec[3]})
    return out
