"""GPU parity over seeded random shapes.

The fixed parity cases pin chosen shapes; this sweep draws shapes at random
(seeded, so every run checks the same ones) across the ranges the launchers
branch on: every token count of the decode product, K from one block to past
the 96-block fused limit (so the split-K rules, the chunk loop and the fused
forms all occur), and N from one 16-row tile to more workgroups than CUs.
Each case runs the decode product (int32 bit-exact, fp32 within the
tolerance), the fused quantise-and-multiply where it applies (bit-identical to
quantise-then-multiply) and, for larger M, the prefill product (bf16 band).
Sizes keep each oracle call to a few tens of millions of multiply-adds."""
import numpy as np
import pytest

import bit_gemv_i2_amd as bn
import oracle
import parity_stats
import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
RTOL = 1e-5
MAX_MACS = 40_000_000


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def draw_shapes(seed, n, m_lo, m_hi):
    r = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(r.integers(m_lo, m_hi + 1))
        nblk = int(r.choice([1, 2, 3, 5, 8, 13, 20, 25, 31, 54, 96, 97, 110]))
        K = 128 * nblk
        tiles = int(r.choice([1, 3, 16, 97, 160, 257, 300, 864]))
        N = 16 * tiles
        if M * N * K <= MAX_MACS:
            out.append((M, N, K))
    return out


def f32_ok(y, ref):
    parity_stats.record(y, ref["y64"], ref["mag"])
    bound = RTOL * np.maximum(np.abs(ref["y64"]), ref["mag"])
    return np.abs(y.astype(np.float64) - ref["y64"]) <= bound


def bf16_ok(ybits, ref):
    tol = RTOL * np.maximum(np.abs(ref["y64"]), ref["mag"])
    lo = wl.bf16_to_f32(oracle.f32_to_bf16((ref["y64"] - tol).astype(np.float32))).astype(np.float64)
    hi = wl.bf16_to_f32(oracle.f32_to_bf16((ref["y64"] + tol).astype(np.float32))).astype(np.float64)
    yv = wl.bf16_to_f32(ybits).astype(np.float64)
    return (yv >= lo) & (yv <= hi)


def fused_fits(M, K):
    return K <= 12288 and M * (K + 16) <= 65280


@pytest.mark.parametrize("M,N,K", draw_shapes(20261203, 28, 1, 16))
def test_decode_random_shapes(gpu, M, N, K):
    c = wl.small_case(M * 131 + N * 7 + K, M, N, K)
    p, st = bn.bitnet_pack_i2s(c.T, c.S)
    pd, sd = dev(p), dev(st)
    xd = dev(c.x_bits.view(np.int16)).view(torch.bfloat16)
    qo, so = oracle.quant_act_bf16(c.x_bits)
    ref = oracle.w2a8(oracle.pack_i2s(c.T), c.S, qo, so, N, K)
    q, s = bn.bitnet_quant_act(xd)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    acc = host(bn.bitnet_w2a8_acc_i32(pd, q, N, K))
    assert np.array_equal(acc, ref["acc"]), f"int32 {M}x{N}x{K}"
    y = host(bn.bitnet_w2a8_gemv(pd, sd, q, s, N, K))
    ok = f32_ok(y, ref)
    assert ok.all(), f"fp32 {M}x{N}x{K}: {(~ok).sum()} outside tolerance"
    if fused_fits(M, K):
        yf = host(bn.bitnet_w2a8_gemv_act(pd, sd, xd, N, K))
        assert np.array_equal(yf.view(np.uint32), y.view(np.uint32)), f"fused {M}x{N}x{K} differs"


@pytest.mark.parametrize("M,N,K", draw_shapes(20261204, 10, 17, 300))
def test_prefill_random_shapes(gpu, M, N, K):
    c = wl.small_case(M * 131 + N * 7 + K, M, N, K)
    p, st = bn.bitnet_pack_i2s(c.T, c.S)
    pd, sd = dev(p), dev(st)
    xd = dev(c.x_bits.view(np.int16)).view(torch.bfloat16)
    qo, so = oracle.quant_act_bf16(c.x_bits)
    ref = oracle.w2a8(oracle.pack_i2s(c.T), c.S, qo, so, N, K)
    q, s = bn.bitnet_quant_act(xd)
    acc = host(bn.bitnet_w2a8_acc_i32(pd, q, N, K))
    assert np.array_equal(acc, ref["acc"]), f"int32 {M}x{N}x{K}"
    y = host(bn.bitnet_w2a8_gemm(pd, sd, q, s, N, K).view(torch.int16)).view(np.uint16)
    ok = bf16_ok(y, ref)
    assert ok.all(), f"bf16 {M}x{N}x{K}: {(~ok).sum()} outside the rounding band"
