"""GPU parity of the scale-granularity variants (64-weight blocks, one scale
per matrix) against the oracle's product for the same format.

Bars as for the 128-block products: the exact int32 sums are shared with the
128 path (the packed weights are the same); fp32 outputs within 1e-5 of
max(|y|, mag); bf16 outputs a round-to-nearest-even of a value inside that
band.  Full-size GEMM outputs are checked on a sample of tokens and rows that
the oracle computes one by one."""
import numpy as np
import pytest

import bit_gemv_i2_amd as bn
import oracle
import parity_stats
import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
RTOL = 1e-5
GRANS = [0, 64]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def close(y, ref, what):
    parity_stats.record(y, ref["y64"], ref["mag"])
    bound = RTOL * np.maximum(np.abs(ref["y64"]), ref["mag"])
    err = np.abs(y.astype(np.float64) - ref["y64"])
    assert not (err > bound).any(), f"{what}: {(err > bound).sum()} outside, worst {(err / bound).max():.3g}x"


def bf16_ok(ybits, ref, what):
    tol = RTOL * np.maximum(np.abs(ref["y64"]), ref["mag"])
    lo = wl.bf16_to_f32(oracle.f32_to_bf16((ref["y64"] - tol).astype(np.float32))).astype(np.float64)
    hi = wl.bf16_to_f32(oracle.f32_to_bf16((ref["y64"] + tol).astype(np.float32))).astype(np.float64)
    yv = wl.bf16_to_f32(ybits).astype(np.float64)
    assert not ((yv < lo) | (yv > hi)).any(), what


def case(seed, G, M, N, K):
    r = wl.rng_for(95, seed, G, M, N, K)
    T = wl.ternary_uniform(r, N, K)
    S = r.uniform(0.5, 2, size=oracle.scale_shape(N, K, G)).astype(np.float32)
    x = r.standard_t(3, size=(M, K)).astype(np.float32)
    q, s = oracle.quant_act_f32(x)
    p, st = bn.bitnet_pack_i2s_g(T, S, G)
    return T, S, q, s, dev(p), dev(st)


SMALL = [(1, 16, 128), (2, 48, 384), (3, 80, 640), (8, 272, 2688), (16, 32, 6912), (5, 64, 12416)]


@pytest.mark.parametrize("G", GRANS)
@pytest.mark.parametrize("M,N,K", SMALL)
def test_gemv_g_matches_oracle(gpu, G, M, N, K):
    T, S, q, s, p, st = case(1, G, M, N, K)
    y = host(bn.bitnet_w2a8_gemv_g(p, st, dev(q), dev(s), N, K, G))
    close(y, oracle.w2a8_g(oracle.pack_i2s_g(T, G), S, q, s, N, K, G), f"gemv_g G={G} {M}x{N}x{K}")


@pytest.mark.parametrize("G", GRANS)
@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (130, 272, 384), (40, 512, 2688), (257, 16, 640)])
def test_gemm_g_matches_oracle(gpu, G, M, N, K):
    T, S, q, s, p, st = case(2, G, M, N, K)
    ref = oracle.w2a8_g(oracle.pack_i2s_g(T, G), S, q, s, N, K, G)
    y32 = host(bn.bitnet_w2a8_gemm_g(p, st, dev(q), dev(s), N, K, G, out_dtype=torch.float32))
    close(y32, ref, f"gemm_g f32 G={G} {M}x{N}x{K}")
    yb = host(bn.bitnet_w2a8_gemm_g(p, st, dev(q), dev(s), N, K, G).view(torch.int16)).view(np.uint16)
    bf16_ok(yb, ref, f"gemm_g bf16 G={G} {M}x{N}x{K}")


def test_g128_entry_points_equal_the_plain_ones(gpu):
    M, N, K = 8, 272, 2688
    T, S, q, s, p, st = case(3, 128, M, N, K)
    qd, sd = dev(q), dev(s)
    a = host(bn.bitnet_w2a8_gemv_g(p, st, qd, sd, N, K, 128))
    b = host(bn.bitnet_w2a8_gemv(p, st, qd, sd, N, K))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    a = host(bn.bitnet_w2a8_gemm_g(p, st, qd, sd, N, K, 128, out_dtype=torch.float32))
    b = host(bn.bitnet_w2a8_gemm(p, st, qd, sd, N, K, out_dtype=torch.float32))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_g0_is_exact_integer_sum_times_scales(gpu):
    # one scale: y = fp32(acc) * (s_a * S), two fp32 roundings of an exact integer
    M, N, K = 4, 96, 2560
    T, S, q, s, p, st = case(4, 0, M, N, K)
    acc = oracle.acc_dense(T, q).astype(np.float32)
    want = acc * (s[:, None] * S[0])
    y = host(bn.bitnet_w2a8_gemv_g(p, st, dev(q), dev(s), N, K, 0))
    assert np.array_equal(y, want)
    y = host(bn.bitnet_w2a8_gemm_g(p, st, dev(q), dev(s), N, K, 0, out_dtype=torch.float32))
    assert np.array_equal(y, want)


@pytest.mark.parametrize("G", GRANS)
@pytest.mark.parametrize("M", [1, 8])
def test_gemv_g_full_config2(gpu, G, M):
    N, K = 13824, 2560
    T, S, q, s, p, st = case(5, G, M, N, K)
    y = host(bn.bitnet_w2a8_gemv_g(p, st, dev(q), dev(s), N, K, G))
    close(y, oracle.w2a8_g(oracle.pack_i2s_g(T, G), S, q, s, N, K, G), f"gemv_g G={G} M={M} full")


@pytest.mark.parametrize("G", GRANS)
def test_gemm_g_full_config4_sampled(gpu, G):
    M, N, K = 512, 13824, 2560
    T, S, q, s, p, st = case(6, G, M, N, K)
    yb = host(bn.bitnet_w2a8_gemm_g(p, st, dev(q), dev(s), N, K, G).view(torch.int16)).view(np.uint16)
    r = wl.rng_for(96, G)
    toks = np.sort(r.choice(M, 12, replace=False))
    rows = np.sort(r.choice(N // 16, 24, replace=False))
    rows = (rows[:, None] * 16 + np.arange(16)).ravel()  # whole 16-row tiles
    Ssub = S if G == 0 else S[rows]
    ref = oracle.w2a8_g(oracle.pack_i2s_g(T[rows], G), Ssub, q[toks], s[toks], rows.size, K, G)
    bf16_ok(yb[np.ix_(toks, rows)], ref, f"gemm_g G={G} full sampled")
