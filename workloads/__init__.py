"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds *inputs only*: shapes, value distributions and seeds.  It
contains none of the method's arithmetic (no ternarisation, packing,
quantisation or product); the oracle and the HIP library each do those on
their own.  The one numeric step here is rounding the generated fp32
activations to bf16 (round-to-nearest-even), because the workloads are
specified as bf16 inputs.

The shapes are those of the pages' GPU latency table ([P2] "5x performance
leap: BitNet vs llama.cpp", section "GPU kernel breakthroughs": 2560x2560,
13824x2560, 20480x3200) and of a ~2.4B-parameter ternary model (hidden 2560,
FFN 6912, 30 layers; [P3] "BitNet + WebAssembly", section "Why WASM", a 2.4B
model of about half a gigabyte at 2 bits per weight).  No trained weights or
datasets are used: every value is drawn from the distribution stated below.

Seeding: ``numpy.random.default_rng(SeedSequence([config, stream, *extra]))``
with stream 0 = weights, 1 = scales, 2 = activations.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK = 128  # weights per scale block (i2_s x86 block)

W_STREAM, S_STREAM, X_STREAM = 0, 1, 2


def rng_for(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- #
# elementary draws
# --------------------------------------------------------------------------- #
def ternary_uniform(rng, N, K) -> np.ndarray:
    """iid {-1,0,+1} with p = 1/3 each, int8 [N][K]."""
    return (rng.integers(0, 3, size=(N, K), dtype=np.int8) - 1).astype(np.int8)


def ternary_choice(rng, N, K, p=(0.3, 0.4, 0.3)) -> np.ndarray:
    """iid {-1,0,+1} with probabilities p, int8 [N][K]."""
    u = rng.random(size=(N, K), dtype=np.float32)
    t = np.zeros((N, K), np.int8)
    t[u < p[0]] = -1
    t[u >= p[0] + p[1]] = 1
    return t


def normal_weights(rng, N, K, std=0.02) -> np.ndarray:
    return (rng.standard_normal(size=(N, K), dtype=np.float32) * np.float32(std)).astype(np.float32)


def uniform_scales(rng, N, K, lo=0.5, hi=2.0, div=1.0) -> np.ndarray:
    s = rng.uniform(lo, hi, size=(N, K // BLOCK)).astype(np.float32)
    if div != 1.0:
        s = (s / np.float32(div)).astype(np.float32)
    return s


def normal_act(rng, M, K) -> np.ndarray:
    return bf16_bits(rng.standard_normal(size=(M, K), dtype=np.float32))


def student_t_act(rng, M, K, dof=3) -> np.ndarray:
    return bf16_bits(rng.standard_t(dof, size=(M, K)).astype(np.float32))


# --------------------------------------------------------------------------- #
# the five workloads
# --------------------------------------------------------------------------- #
@dataclass
class Case:
    """One product workload.  Exactly one of (T, W) is set: T is a ternary
    matrix with scales S; W is an fp32 matrix still to be ternarised
    (absmean, per 128-block) by whoever consumes it."""
    name: str
    M: int
    N: int
    K: int
    x_bits: np.ndarray            # bf16 bit patterns [M][K]
    T: np.ndarray | None = None   # int8 [N][K]
    S: np.ndarray | None = None   # fp32 [N][K/128]
    W: np.ndarray | None = None   # fp32 [N][K]
    meta: dict = field(default_factory=dict)


def config1(M=1, seed=0) -> Case:
    """2560x2560 GEMV: iid uniform ternary, scales U[0.5,2], x ~ N(0,1) bf16."""
    N = K = 2560
    return Case("gemv_2560x2560", M, N, K,
                x_bits=normal_act(rng_for(1, X_STREAM, seed, M), M, K),
                T=ternary_uniform(rng_for(1, W_STREAM, seed), N, K),
                S=uniform_scales(rng_for(1, S_STREAM, seed), N, K))


def config2(M=1, seed=0) -> Case:
    """13824x2560 GEMV (fused FFN gate+up shape): W ~ N(0, 0.02) fp32, to be
    absmean-ternarised per block; x ~ N(0,1) bf16."""
    N, K = 13824, 2560
    return Case("gemv_13824x2560", M, N, K,
                x_bits=normal_act(rng_for(2, X_STREAM, seed, M), M, K),
                W=normal_weights(rng_for(2, W_STREAM, seed), N, K, 0.02))


def config3(M=1, seed=0) -> Case:
    """20480x3200 GEMV: P(-1,0,+1) = (.3,.4,.3), scales U[0.5,2], x ~ Student-t(3) bf16."""
    N, K = 20480, 3200
    return Case("gemv_20480x3200", M, N, K,
                x_bits=student_t_act(rng_for(3, X_STREAM, seed, M), M, K),
                T=ternary_choice(rng_for(3, W_STREAM, seed), N, K),
                S=uniform_scales(rng_for(3, S_STREAM, seed), N, K))


def config4(M=512, seed=0) -> Case:
    """Prefill GEMM 512 x 13824 x 2560: uniform ternary, scales U[0.5,2], X ~ N(0,1) bf16."""
    N, K = 13824, 2560
    return Case("gemm_512x13824x2560", M, N, K,
                x_bits=normal_act(rng_for(4, X_STREAM, seed, M), M, K),
                T=ternary_uniform(rng_for(4, W_STREAM, seed), N, K),
                S=uniform_scales(rng_for(4, S_STREAM, seed), N, K))


# Decode stack of a ~2.4B ternary model: per layer four 2560x2560 projections,
# one fused 13824x2560 gate+up and one 2560x6912 down projection.
STACK_HIDDEN = 2560
STACK_FFN = 6912
STACK_LAYERS = 30
STACK_SHAPES = [(2560, 2560)] * 4 + [(2 * STACK_FFN, STACK_HIDDEN), (STACK_HIDDEN, STACK_FFN)]


def stack_matrix(layer: int, idx: int, seed=0):
    """(T int8 [N][K], S fp32 [N][K/128]) of matrix idx (0..5) of a layer:
    uniform ternary, scales U[0.5,2] / sqrt(7K/6) so that the rms gain of one
    product is about 1 and the chain neither grows nor vanishes."""
    N, K = STACK_SHAPES[idx]
    T = ternary_uniform(rng_for(5, W_STREAM, seed, layer, idx), N, K)
    S = uniform_scales(rng_for(5, S_STREAM, seed, layer, idx), N, K, div=math.sqrt(7.0 * K / 6.0))
    return T, S


def stack_input(M=1, seed=0) -> np.ndarray:
    return normal_act(rng_for(5, X_STREAM, seed, M), M, STACK_HIDDEN)


def small_case(seed, M, N, K, wkind="uniform", xkind="normal", skind="uniform") -> Case:
    """Small seeded case for parity tests (several tiles plus ragged tails)."""
    rw, rs, rx = rng_for(100, W_STREAM, seed, M, N, K), rng_for(100, S_STREAM, seed, M, N, K), \
        rng_for(100, X_STREAM, seed, M, N, K)
    c = Case(f"small_{M}x{N}x{K}_s{seed}", M, N, K, x_bits=None)
    if wkind == "uniform":
        c.T = ternary_uniform(rw, N, K)
    elif wkind == "sparse":
        c.T = ternary_choice(rw, N, K, (0.3, 0.4, 0.3))
    elif wkind == "normal":
        c.W = normal_weights(rw, N, K, 0.02)
    else:
        raise ValueError(wkind)
    if c.T is not None:
        c.S = uniform_scales(rs, N, K) if skind == "uniform" else np.ones((N, K // BLOCK), np.float32)
    c.x_bits = normal_act(rx, M, K) if xkind == "normal" else student_t_act(rx, M, K)
    return c


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4}
