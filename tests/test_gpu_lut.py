"""GPU parity of the table-lookup decode product (bitnet_w2a8_gemv_lut)
against the CPU oracle: int32 sums bit-exact, fp32 outputs within 1e-5 of
max(|y|, s_a * sum_b |S*A|), for every tiles-per-workgroup choice; and equal
integer sums to the matrix-core decode kernel on the same operands."""
import numpy as np
import pytest

import bit_gemv_i2_amd as bn
import oracle
import parity_stats
import workloads as wl

pytestmark = pytest.mark.gpu
RTOL = 1e-5

torch = pytest.importorskip("torch")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check(T, S, q, s_a, tiles, what):
    N, K = T.shape
    ref = oracle.w2a8(oracle.pack_i2s(T), S, q, s_a, N, K)
    p, st = bn.bitnet_pack_i2s(T, S)
    y, acc = bn.bitnet_w2a8_gemv_lut(dev(p), dev(st), dev(q), dev(s_a), N, K, tiles, with_acc=True)
    assert np.array_equal(host(acc), ref["acc"]), f"{what}: int32 sums differ"
    parity_stats.record(host(y), ref["y64"], ref["mag"])
    bound = RTOL * np.maximum(np.abs(ref["y64"]), ref["mag"])
    err = np.abs(host(y).astype(np.float64) - ref["y64"])
    assert not (err > bound).any(), f"{what}: {(err > bound).sum()} outputs outside tolerance"


# several tiles and blocks, ragged tile groups (N/16 not a multiple of 4) and
# ragged wave slices (blocks not a multiple of the waves)
SHAPES = [(16, 128), (48, 384), (80, 640), (272, 2688), (64, 8960), (2064, 384), (208, 3200), (1040, 2560)]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("tiles", [0, 1, 2, 4])
def test_lut_gemv_small(gpu, N, K, tiles):
    c = wl.small_case(N * 3 + K + tiles, 1, N, K, xkind="t3", wkind="sparse")
    q, s = oracle.quant_act_bf16(c.x_bits)
    check(c.T, c.S, q, s, tiles, f"{N}x{K} tiles={tiles}")


def test_lut_gemv_extreme_codes(gpu):
    # every code pair of every table entry: all -1, all +1, alternating signs,
    # and activations at both ends of the int8 range (|entry| up to 254)
    N, K = 64, 512
    T = np.ones((N, K), np.int8)
    T[16:32] = -1
    T[32:48, 0::2] = -1
    T[48:64] = 0
    T[48:64, 5::7] = 1
    q = np.where(np.arange(K) % 3 == 0, 127, -127).astype(np.int8)[None, :]
    q[0, 1::4] = -128 + 1
    s_a = np.array([0.5], np.float32)
    S = np.full((N, K // 128), 1.25, np.float32)
    for tiles in (1, 4):
        check(T, S, q, s_a, tiles, f"extreme tiles={tiles}")


def test_lut_gemv_matches_matrix_core_integer_sums(gpu):
    c = wl.config2(M=1)
    T, S = bn.bitnet_ternarize_absmean(c.W)
    q, s = oracle.quant_act_bf16(c.x_bits)
    p, st = bn.bitnet_pack_i2s(T, S)
    pd, sd, qd, sa = dev(p), dev(st), dev(q), dev(s)
    acc_mc = host(bn.bitnet_w2a8_acc_i32(pd, qd, c.N, c.K))
    for tiles in (1, 2, 4):
        _, acc = bn.bitnet_w2a8_gemv_lut(pd, sd, qd, sa, c.N, c.K, tiles, with_acc=True)
        assert np.array_equal(host(acc), acc_mc), f"tiles={tiles}"


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [1, 3])
def test_lut_gemv_full_configs(gpu, cfg):
    c = wl.config1() if cfg == 1 else wl.config3()
    q, s = oracle.quant_act_bf16(c.x_bits)
    check(c.T, c.S, q, s, 0, f"config{cfg}")
