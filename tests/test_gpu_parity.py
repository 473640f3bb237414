"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bars: int8 activations, dequant factors and int32 accumulators bit-exact;
fp32 outputs within 1e-5 of max(|y|, mag) where mag = s_a * sum_b |S*A| (the
epilogue's fp32 summation order is free; its worst-case rounding is about
(blocks + waves) * 2^-24 * mag); bf16 outputs are a round-to-nearest-even of a
value inside that band."""
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


def x_dev(bits):
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def pack_dev(T, S):
    p, s = bn.bitnet_pack_i2s(T, S)
    return dev(p), dev(s)


def assert_f32_close(y, ref, what=""):
    y64, mag = ref["y64"], ref["mag"]
    parity_stats.record(y, y64, mag)
    bound = RTOL * np.maximum(np.abs(y64), mag)
    err = np.abs(y.astype(np.float64) - y64)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} outside tolerance, worst {(err / np.maximum(bound, 1e-300)).max():.3g}x"


def assert_bf16_ok(ybits, ref, what=""):
    y64, mag = ref["y64"], ref["mag"]
    tol = RTOL * np.maximum(np.abs(y64), mag)
    lo = wl.bf16_to_f32(oracle.f32_to_bf16((y64 - tol).astype(np.float32))).astype(np.float64)
    hi = wl.bf16_to_f32(oracle.f32_to_bf16((y64 + tol).astype(np.float32))).astype(np.float64)
    yv = wl.bf16_to_f32(ybits).astype(np.float64)
    bad = (yv < lo) | (yv > hi)
    assert not bad.any(), f"{what}: {bad.sum()} bf16 outputs outside the rounding band"


def oracle_ref(T, S, q, s_a):
    N, K = T.shape
    return oracle.w2a8(oracle.pack_i2s(T), S, q, s_a, N, K)


# ------------------------------------------------------------------ MFMA operand layout (builtin check)
def test_zz_layout_single_weight(gpu):
    # one nonzero weight at a time, one nonzero activation: checks every index of the decode
    N, K = 32, 256
    for (n, k) in [(0, 0), (17, 130), (31, 255), (5, 64 + 48 + 9), (16, 7), (9, 127)]:
        T = np.zeros((N, K), np.int8)
        T[n, k] = -1
        q = np.zeros((3, K), np.int8)
        q[2, k] = 101
        q[0, k] = -7
        p, s = pack_dev(T, np.ones((N, K // 128), np.float32))
        acc = host(bn.bitnet_w2a8_acc_i32(p, dev(q), N, K))
        want = np.zeros((3, N), np.int32)
        want[2, n] = -101
        want[0, n] = 7
        assert np.array_equal(acc, want), (n, k)


# ------------------------------------------------------------------ activation quantisation
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_quant_bf16_configs_bitexact(gpu, cfg):
    M = {1: 1, 2: 8, 3: 1, 4: 512}[cfg]
    c = wl.CONFIGS[cfg](M=M)
    q, s = bn.bitnet_quant_act(x_dev(c.x_bits))
    qo, so = oracle.quant_act_bf16(c.x_bits)
    assert np.array_equal(host(q), qo)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("M,K", [(1, 16), (3, 2576), (7, 6912), (2, 4096 + 16)])
def test_quant_f32_and_edge_bitexact(gpu, M, K):
    r = wl.rng_for(51, M, K)
    x = (r.standard_t(3, size=(M, K)) * 10.0 ** r.integers(-3, 4, size=(M, 1))).astype(np.float32)
    x[0] = 0.0  # zero token -> q = 0, s_a = 1e-5/127
    if M > 1:
        x[1, ::7] = -x[1, ::7]
    q, s = bn.bitnet_quant_act(dev(x))
    qo, so = oracle.quant_act_f32(x)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    assert np.all(host(q)[0] == 0)


def tie_activations(M, K, seed):
    """Activations whose every scaled value x * inv is an exact half-integer: even tokens
    hold half-integers with amax 127 (inv = 1), odd tokens odd integers with amax 254
    (inv = 0.5).  All are exact in bf16 as well as fp32."""
    r = wl.rng_for(seed, M, K)
    x = np.empty((M, K), np.float32)
    for m in range(M):
        if m % 2 == 0:
            x[m] = r.integers(-127, 127, size=K) + 0.5
            x[m, m % K] = 127.0
        else:
            x[m] = 2 * r.integers(-127, 127, size=K) + 1
            x[m, m % K] = -254.0
    return x


# Round half to even on exact ties, in the standalone quantiser and in every fused form:
# quantise-first (13824 rows), all waves (272 rows), busiest-SIMD split (2560 x 1280) and
# the extra quant waves (8 tokens).
@pytest.mark.parametrize("M,N,K", [(1, 13824, 2560), (2, 272, 2688), (1, 2560, 1280), (8, 2064, 2560)])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_quant_exact_ties_round_half_to_even(gpu, xdt, M, N, K):
    x = tie_activations(M, K, 73)
    if xdt == "bf16":
        bits = wl.bf16_bits(x)
        assert np.array_equal(wl.bf16_to_f32(bits), x)
        xd = x_dev(bits)
        qo, so = oracle.quant_act_bf16(bits)
    else:
        xd = dev(x)
        qo, so = oracle.quant_act_f32(x)
    ties = np.ones((M, K), bool)
    ties[np.arange(M), np.arange(M) % K] = False
    assert np.all(qo[ties] % 2 == 0) and np.all(np.abs(qo[~ties]) == 127)
    q, s = bn.bitnet_quant_act(xd)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    c = wl.small_case(M * 7 + N + K, M, N, K)
    p, st = pack_dev(c.T, c.S)
    q_out = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s_out = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = bn.bitnet_w2a8_gemv_act(p, st, xd, N, K, q_out=q_out, s_a_out=s_out)
    assert np.array_equal(host(q_out), qo) and np.array_equal(host(s_out), so)
    assert_f32_close(host(y), oracle_ref(c.T, c.S, qo, so), f"ties {xdt} {M}x{N}x{K}")


@pytest.mark.parametrize("M,H", [(1, 6912), (8, 6912), (3, 48)])
def test_quant_fold_bitexact(gpu, M, H):
    y = wl.rng_for(52, M, H).standard_normal((M, 2 * H)).astype(np.float32) * 3
    q, s = bn.bitnet_quant_act_fold(dev(y))
    qo, so = oracle.fold_quant(y)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)


@pytest.mark.parametrize("M,H", [(1, 6912), (8, 6912), (3, 48)])
def test_quant_relu2_glu_bitexact(gpu, M, H):
    y = wl.rng_for(53, M, H).standard_normal((M, 2 * H)).astype(np.float32) * 3
    if M > 1:
        y[1, :H] = -np.abs(y[1, :H])  # every gate negative -> zero token
    q, s = bn.bitnet_quant_act_relu2_glu(dev(y))
    qo, so = oracle.glu_quant(y)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    if M > 1:
        assert not np.any(host(q)[1])


# ------------------------------------------------------------------ exact integer core
SMALL_SHAPES = [(16, 128), (48, 384), (80, 640), (272, 2688), (64, 8960), (2064, 128 * 3)]


@pytest.mark.parametrize("N,K", SMALL_SHAPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 16])
def test_acc_i32_gemv_path_bitexact(gpu, M, N, K):
    c = wl.small_case(M * 7 + N, M, N, K)
    q, s = oracle.quant_act_bf16(c.x_bits)
    p, st = pack_dev(c.T, c.S)
    acc = host(bn.bitnet_w2a8_acc_i32(p, dev(q), N, K))
    assert np.array_equal(acc, oracle_ref(c.T, c.S, q, s)["acc"])


@pytest.mark.parametrize("M,N,K", [(17, 48, 384), (130, 272, 1280), (300, 160, 2560), (512, 16, 128)])
def test_acc_i32_gemm_path_bitexact(gpu, M, N, K):
    c = wl.small_case(M + N + K, M, N, K, wkind="sparse")
    q, s = oracle.quant_act_bf16(c.x_bits)
    p, st = pack_dev(c.T, c.S)
    acc = host(bn.bitnet_w2a8_acc_i32(p, dev(q), N, K))
    assert np.array_equal(acc, oracle_ref(c.T, c.S, q, s)["acc"])


# ------------------------------------------------------------------ fp32 / bf16 products
@pytest.mark.parametrize("N,K", SMALL_SHAPES)
@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_gemv_small_within_tolerance(gpu, M, N, K):
    c = wl.small_case(M * 11 + K, M, N, K, xkind="t3")
    q, s = oracle.quant_act_bf16(c.x_bits)
    p, st = pack_dev(c.T, c.S)
    y = host(bn.bitnet_w2a8_gemv(p, st, dev(q), dev(s), N, K))
    assert_f32_close(y, oracle_ref(c.T, c.S, q, s), f"gemv {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 48, 384), (33, 272, 1280), (130, 160, 2688), (256, 144, 640)])
@pytest.mark.parametrize("ydt", ["bf16", "f32"])
def test_gemm_small_within_tolerance(gpu, M, N, K, ydt):
    c = wl.small_case(M * 3 + N, M, N, K)
    q, s = oracle.quant_act_bf16(c.x_bits)
    p, st = pack_dev(c.T, c.S)
    out = torch.bfloat16 if ydt == "bf16" else torch.float32
    y = bn.bitnet_w2a8_gemm(p, st, dev(q), dev(s), N, K, out_dtype=out)
    ref = oracle_ref(c.T, c.S, q, s)
    if ydt == "bf16":
        assert_bf16_ok(host(y.view(torch.int16)).view(np.uint16), ref, "gemm bf16")
    else:
        assert_f32_close(host(y), ref, "gemm f32")


def test_zero_weights_and_zero_tokens(gpu):
    M, N, K = 4, 64, 1024
    c = wl.small_case(3, M, N, K)
    x = wl.bf16_to_f32(c.x_bits)
    x[2] = 0.0
    q, s = bn.bitnet_quant_act(dev(x))
    p, st = pack_dev(c.T, c.S)
    y = host(bn.bitnet_w2a8_gemv(p, st, q, s, N, K))
    assert np.all(y[2] == 0.0)
    pz, sz = pack_dev(np.zeros((N, K), np.int8), c.S)
    assert np.all(host(bn.bitnet_w2a8_gemv(pz, sz, q, s, N, K)) == 0.0)
    assert np.all(host(bn.bitnet_w2a8_gemm(pz, sz, q, s, N, K, out_dtype=torch.float32)) == 0.0)


# ------------------------------------------------------------------ fused quantise-and-multiply
@pytest.mark.parametrize("mode", ["bf16", "f32", "fold", "relu2_glu"])
@pytest.mark.parametrize("M,N,K", [(1, 48, 384), (2, 272, 2688), (3, 80, 640), (5, 160, 6912), (8, 2064, 2560),
                                   (16, 32, 128), (1, 64, 12288),
                                   # more 16-row workgroups than CUs: the quantise-first form
                                   (1, 4112, 384), (2, 6912, 2560),
                                   # at most one workgroup per CU: busiest-SIMD splits
                                   # (waves x blocks 4x7, 4x3, 4x5)
                                   (1, 2560, 3200), (1, 2560, 1280), (8, 2560, 2560)])
def test_gemv_act_matches_oracle_and_unfused(gpu, mode, M, N, K):
    c = wl.small_case(M * 5 + N + K, M, N, K, xkind="t3")
    p, st = pack_dev(c.T, c.S)
    if mode == "bf16":
        xd = x_dev(c.x_bits)
        qo, so = oracle.quant_act_bf16(c.x_bits)
        qd, sd = bn.bitnet_quant_act(xd)
    else:
        x = wl.bf16_to_f32(c.x_bits) * np.float32(0.37)
        if mode in ("fold", "relu2_glu"):
            x = np.concatenate([x, wl.rng_for(61, M, K).standard_normal((M, K)).astype(np.float32)], axis=1)
            xd = dev(x)
            if mode == "fold":
                qo, so = oracle.fold_quant(x)
                qd, sd = bn.bitnet_quant_act_fold(xd)
            else:
                qo, so = oracle.glu_quant(x)
                qd, sd = bn.bitnet_quant_act_relu2_glu(xd)
        else:
            qo, so = oracle.quant_act_f32(x)
            xd = dev(x)
            qd, sd = bn.bitnet_quant_act(xd)
    q_out = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s_out = torch.empty((M,), dtype=torch.float32, device="cuda")
    junction = {"fold": "sum", "relu2_glu": "relu2_glu"}.get(mode, False)
    y = bn.bitnet_w2a8_gemv_act(p, st, xd, N, K, fold=junction, q_out=q_out, s_a_out=s_out)
    y_ref = bn.bitnet_w2a8_gemv(p, st, qd, sd, N, K)
    assert np.array_equal(host(q_out), qo) and np.array_equal(host(s_out), so)
    yh = host(y)
    assert np.array_equal(yh.view(np.uint32), host(y_ref).view(np.uint32)), "fused and unfused differ"
    assert_f32_close(yh, oracle_ref(c.T, c.S, qo, so), f"gemv_act {mode} {M}x{N}x{K}")


# With more 16-row workgroups than CUs (all resident), the fused step takes the form that
# quantises before requesting the weights; same arithmetic, so bit-identical to the unfused path.
# 20480x3200 takes 5 waves of 5 blocks (the split that keeps all 1280 workgroups resident).
@pytest.mark.parametrize("M,N,K", [(1, 4112, 384), (2, 6912, 2560), (1, 13824, 2560), (4, 9216, 1280),
                                   (1, 20480, 3200), (2, 20480, 3200)])
def test_gemv_act_quantise_first_form_bitexact(gpu, M, N, K):
    assert N // 16 > torch.cuda.get_device_properties(0).multi_processor_count
    c = wl.small_case(M * 7 + N + K, M, N, K, xkind="t3")
    p, st = pack_dev(c.T, c.S)
    xd = x_dev(c.x_bits)
    qo, so = oracle.quant_act_bf16(c.x_bits)
    qd, sd = bn.bitnet_quant_act(xd)
    q_out = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s_out = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = host(bn.bitnet_w2a8_gemv_act(p, st, xd, N, K, q_out=q_out, s_a_out=s_out))
    y_ref = host(bn.bitnet_w2a8_gemv(p, st, qd, sd, N, K))
    assert np.array_equal(host(q_out), qo) and np.array_equal(host(s_out), so)
    assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32)), "fused and unfused differ"
    assert_f32_close(y, oracle_ref(c.T, c.S, qo, so), f"gemv_act quantise-first {M}x{N}x{K}")


def test_gemv_act_rejects_what_does_not_fit(gpu):
    # M*K beyond the LDS copy of q, and K beyond 12 waves x 8 blocks
    for (M, K) in [(16, 8192), (1, 12288 + 128)]:
        p, st = pack_dev(np.zeros((16, K), np.int8), np.ones((16, K // 128), np.float32))
        x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(bn.BitnetError) as ei:
            bn.bitnet_w2a8_gemv_act(p, st, x, 16, K)
        assert ei.value.status == bn.BITNET_ERR_UNSUPPORTED_SHAPE


# ------------------------------------------------------------------ full-size workloads
def _full_gemv(c, T, S, what):
    # end to end on the device: bf16 activations -> quant -> product
    qd, sd = bn.bitnet_quant_act(x_dev(c.x_bits))
    qo, so = oracle.quant_act_bf16(c.x_bits)
    assert np.array_equal(host(qd), qo) and np.array_equal(host(sd), so)
    p, st = pack_dev(T, S)
    y = host(bn.bitnet_w2a8_gemv(p, st, qd, sd, c.N, c.K))
    ref = oracle_ref(T, S, qo, so)
    assert_f32_close(y, ref, what)
    acc = host(bn.bitnet_w2a8_acc_i32(p, qd, c.N, c.K))
    assert np.array_equal(acc, ref["acc"])


@pytest.mark.slow
def test_config1_gemv_full(gpu):
    c = wl.config1()
    _full_gemv(c, c.T, c.S, "config1")


@pytest.mark.slow
@pytest.mark.parametrize("M", [1, 8])
def test_config2_gemv_full(gpu, M):
    c = wl.config2(M=M)
    T, S = bn.bitnet_ternarize_absmean(c.W)
    To, So = oracle.ternarize_absmean(c.W)
    assert np.array_equal(T, To) and np.array_equal(S, So)
    _full_gemv(c, T, S, f"config2 M={M}")


@pytest.mark.slow
def test_config3_gemv_full(gpu):
    c = wl.config3()
    _full_gemv(c, c.T, c.S, "config3")


@pytest.mark.slow
@pytest.mark.parametrize("idx", [0, 4, 5])
@pytest.mark.parametrize("M", [1, 8])
def test_stack_shapes_gemv_full(gpu, idx, M):
    T, S = wl.stack_matrix(0, idx)
    N, K = T.shape
    xb = wl.normal_act(wl.rng_for(53, idx, M), M, K)
    c = wl.Case(f"stack{idx}", M, N, K, x_bits=xb)
    _full_gemv(c, T, S, f"stack matrix {idx} M={M}")


@pytest.mark.slow
def test_config4_gemm_full(gpu):
    """The whole 512 x 13824 output of the prefill workload (int32 sums, bf16 and fp32
    results) against the oracle, which runs its rows in a process pool."""
    import oracle_pool as op
    c = wl.config4()
    qd, sd = bn.bitnet_quant_act(x_dev(c.x_bits))
    qo, so = oracle.quant_act_bf16(c.x_bits)
    assert np.array_equal(host(qd), qo) and np.array_equal(host(sd), so)
    p, st = pack_dev(c.T, c.S)
    ybits = host(bn.bitnet_w2a8_gemm(p, st, qd, sd, c.N, c.K).view(torch.int16)).view(np.uint16)
    y32 = host(bn.bitnet_w2a8_gemm(p, st, qd, sd, c.N, c.K, out_dtype=torch.float32))
    acc = host(bn.bitnet_w2a8_acc_i32(p, qd, c.N, c.K))
    step = 432
    print(f"config4: oracle on {c.M} x {c.N} outputs in {op.workers()} processes", flush=True)
    seen = 0
    worst = plain = 0.0
    with op.pool() as ex:
        for n0, acc_o, y64, mag in ex.map(op.config4_rows, range(0, c.N, step), range(step, c.N + step, step)):
            n1 = n0 + acc_o.shape[1]
            ref = {"y64": y64, "mag": mag}
            assert np.array_equal(acc[:, n0:n1], acc_o), f"int32 sums differ in rows {n0}..{n1}"
            assert_bf16_ok(ybits[:, n0:n1], ref, f"config4 bf16 rows {n0}..{n1}")
            assert_f32_close(y32[:, n0:n1], ref, f"config4 f32 rows {n0}..{n1}")
            r, _, pl = op.f32_check(y32[:, n0:n1], y64, mag)
            worst, plain = max(worst, r), max(plain, pl)
            seen += n1 - n0
    assert seen == c.N
    print(f"config4: every output checked; fp32 worst error / bound {worst:.3f}, plain max relative error {plain:.3e}")


# ------------------------------------------------------------------ prefill row-tile choices
# Few-token launches use narrower workgroup tiles (256 -> 128 -> 64 rows) so that the
# grid still fills the chip: 64 x 13824 and 512 x 2560 take 64-row tiles, 256 x 13824
# takes 128-row tiles, 512 x 13824 the full 256 rows.
# 64-token tiles with two blocks per pipeline stage (up to 128 tokens, or few workgroups: 512 x
# 2560 x 6912 runs 8 of them x 40 row groups), with 1 row tile per wave (64, 40, 130 tokens) and
# with 2 (26624 / 30736 rows, and 100 tokens x 13824 rows), odd block counts and ragged token
# tiles included; 256 tokens x 13824 rows keeps the 128-token tiles
@pytest.mark.parametrize("M,N,K", [(64, 13824, 2560), (256, 13824, 2560), (512, 2560, 6912), (40, 2576, 640),
                                   (48, 26624, 384), (17, 30736, 1152), (64, 26624, 2560), (100, 13824, 640),
                                   (130, 2560, 1152)])
def test_gemm_row_tile_choices_sampled(gpu, M, N, K):
    c = wl.small_case(M + N + K, M, N, K)
    p, st = pack_dev(c.T, c.S)
    qd, sd = bn.bitnet_quant_act(x_dev(c.x_bits))
    qo, so = oracle.quant_act_bf16(c.x_bits)
    yb = host(bn.bitnet_w2a8_gemm(p, st, qd, sd, N, K).view(torch.int16)).view(np.uint16)
    y32 = host(bn.bitnet_w2a8_gemm(p, st, qd, sd, N, K,
                                   y=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")))
    acc = host(bn.bitnet_w2a8_acc_i32(p, qd, N, K))
    r = wl.rng_for(97, M, N, K)
    toks = np.sort(r.choice(M, min(M, 12), replace=False))
    tiles = np.sort(r.choice(N // 16, min(N // 16, 16), replace=False))
    rows = (tiles[:, None] * 16 + np.arange(16)).ravel()
    ref = oracle.w2a8(oracle.pack_i2s(c.T[rows]), c.S[rows], qo[toks], so[toks], rows.size, K)
    assert np.array_equal(acc[np.ix_(toks, rows)], ref["acc"])
    assert_f32_close(y32[np.ix_(toks, rows)], ref, f"gemm f32 {M}x{N}x{K}")
    assert_bf16_ok(yb[np.ix_(toks, rows)], ref, f"gemm bf16 {M}x{N}x{K}")
    # every output element is written (the buffer started as NaN)
    assert np.isfinite(y32).all()


# ------------------------------------------------------------------ the 256-row form on ragged shapes
# A launch with at least 200 workgroups of 128 tokens x 256 rows runs the 256-row kernel
# (weights and activations loaded straight into a ring of four LDS stages, matrix-core
# steps interleaved with the drain).  These shapes reach it with a partial last token tile,
# a partial last 256-row group (clamped weight loads, stores cut at N) and 1, 2, 3 and 5
# K-blocks (with one block every prefetch repeats block 0; at five the ring wraps).
def wide_form(M, N):
    return -(-M // 128) * -(-N // 256) >= 200


def edge_samples(r, M, N):
    toks = {0, M - 1, (M // 128) * 128 % M} | set(r.choice(M, 10, replace=False).tolist())
    tiles = {0, N // 16 - 1, (N // 256) * 16 % (N // 16)} | set(r.choice(N // 16, 12, replace=False).tolist())
    toks, tiles = np.array(sorted(toks)), np.array(sorted(tiles))
    return toks, (tiles[:, None] * 16 + np.arange(16)).ravel()


@pytest.mark.parametrize("M,N,K", [(3207, 2064, 384), (1700, 4112, 128), (2000, 3328, 640), (1000, 6400, 256)])
def test_gemm_wide_form_ragged_sampled(gpu, M, N, K):
    assert wide_form(M, N)
    c = wl.small_case(M + N + K, M, N, K)
    p, st = pack_dev(c.T, c.S)
    qd, sd = bn.bitnet_quant_act(x_dev(c.x_bits))
    qo, so = oracle.quant_act_bf16(c.x_bits)
    yb = host(bn.bitnet_w2a8_gemm(p, st, qd, sd, N, K, y=torch.full((M, N), float("nan"), dtype=torch.bfloat16,
                                                                    device="cuda")).view(torch.int16)).view(np.uint16)
    y32 = host(bn.bitnet_w2a8_gemm(p, st, qd, sd, N, K,
                                   y=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")))
    acc = host(bn.bitnet_w2a8_acc_i32(p, qd, N, K))
    toks, rows = edge_samples(wl.rng_for(98, M, N, K), M, N)
    ref = oracle.w2a8(oracle.pack_i2s(c.T[rows]), c.S[rows], qo[toks], so[toks], rows.size, K)
    assert np.array_equal(acc[np.ix_(toks, rows)], ref["acc"])
    assert_f32_close(y32[np.ix_(toks, rows)], ref, f"wide f32 {M}x{N}x{K}")
    assert_bf16_ok(yb[np.ix_(toks, rows)], ref, f"wide bf16 {M}x{N}x{K}")
    # every output element is written (both buffers started as NaN)
    assert np.isfinite(y32).all() and np.isfinite(wl.bf16_to_f32(yb)).all()


@pytest.mark.parametrize("M,N,K", [(3207, 2064, 384), (1700, 4112, 128)])
def test_gemm_wide_form_one_scale_ragged_sampled(gpu, M, N, K):
    assert wide_form(M, N)
    c = wl.small_case(M + N + K + 1, M, N, K)
    S0 = np.array([0.75], np.float32)
    p, st = bn.bitnet_pack_i2s_g(c.T, S0, 0)
    p, st = dev(p), dev(st)
    qd, sd = bn.bitnet_quant_act(x_dev(c.x_bits))
    qo, so = oracle.quant_act_bf16(c.x_bits)
    y32 = host(bn.bitnet_w2a8_gemm_g(p, st, qd, sd, N, K, 0, out_dtype=torch.float32))
    yb = host(bn.bitnet_w2a8_gemm_g(p, st, qd, sd, N, K, 0).view(torch.int16)).view(np.uint16)
    toks, rows = edge_samples(wl.rng_for(99, M, N, K), M, N)
    ref = oracle.w2a8_g(oracle.pack_i2s_g(c.T[rows], 0), S0, qo[toks], so[toks], rows.size, K, 0)
    assert_f32_close(y32[np.ix_(toks, rows)], ref, f"wide G=0 f32 {M}x{N}x{K}")
    assert_bf16_ok(yb[np.ix_(toks, rows)], ref, f"wide G=0 bf16 {M}x{N}x{K}")


# ------------------------------------------------------------------ the largest K
def test_max_k_integer_sums_do_not_overflow(gpu):
    # the int32 accumulators hold 64 x the integer sum: at the largest K with every
    # weight +1 and every activation 127 the sum is 127 * 262144 = 33,292,288 and
    # 64 x that = 2,130,706,432 < 2^31; one block more is rejected
    K = 262144
    N, M = 16, 2
    T = np.ones((N, K), np.int8)
    T[1::2] = -1
    p, st = pack_dev(T, np.ones((N, K // 128), np.float32))
    q = np.full((M, K), 127, np.int8)
    q[1] = -127
    qd = dev(q)
    acc = host(bn.bitnet_w2a8_acc_i32(p, qd, N, K))
    want = np.where(np.arange(N)[None, :] % 2 == 0, 1, -1) * np.array([[127], [-127]]) * K
    assert np.array_equal(acc, want.astype(np.int32))
    # the fp32 product through the same kernels: unit scales, s_a = 1 -> y == acc exactly
    y = host(bn.bitnet_w2a8_gemv(p, st, qd, dev(np.ones(M, np.float32)), N, K))
    assert np.array_equal(y, want.astype(np.float32))
    pb, sb = pack_dev(np.ones((N, K + 128), np.int8), np.ones((N, (K + 128) // 128), np.float32))
    with pytest.raises(bn.BitnetError) as ei:
        bn.bitnet_w2a8_acc_i32(pb, dev(np.ones((M, K + 128), np.int8)), N, K + 128)
    assert ei.value.status == bn.BITNET_ERR_UNSUPPORTED_SHAPE


# ------------------------------------------------------------------ the largest grids
# 2^20 rows (65,536 decode workgroups; 4,096 workgroups of the 256-row prefill kernel at 40
# tokens), K of one and two blocks: sampled rows at both ends and in between
@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (40, 128)])
def test_tall_matrix_grids_sampled(gpu, M, K):
    N = 1 << 20
    r = wl.rng_for(131, M, K)
    T = wl.ternary_uniform(r, N, K)
    S = wl.uniform_scales(r, N, K)
    xb = wl.normal_act(r, M, K)
    p, st = pack_dev(T, S)
    qd, sd = bn.bitnet_quant_act(x_dev(xb))
    qo, so = oracle.quant_act_bf16(xb)
    acc = host(bn.bitnet_w2a8_acc_i32(p, qd, N, K))
    y = host(bn.bitnet_w2a8_gemv(p, st, qd, sd, N, K)) if M <= 16 else \
        host(bn.bitnet_w2a8_gemm(p, st, qd, sd, N, K, out_dtype=torch.float32))
    tiles = np.unique(np.concatenate([[0, 1, N // 32, N // 16 - 2, N // 16 - 1], r.choice(N // 16, 24)]))
    rows = (tiles[:, None] * 16 + np.arange(16)).ravel()
    ref = oracle.w2a8(oracle.pack_i2s(T[rows]), S[rows], qo, so, rows.size, K)
    assert np.array_equal(acc[:, rows], ref["acc"])
    assert_f32_close(y[:, rows], ref, f"tall {M}x{N}x{K}")


# ------------------------------------------------------------------ measurement helper
@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 10_011_152])
def test_stream_read_probe_reads_every_word(gpu, nbytes):
    # the benchmark's bare-stream reference must really read the whole buffer once
    words = wl.rng_for(98, nbytes).integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    sink = host(bn.bitnet_probe_stream_read(dev(words.view(np.int32))))
    assert int(sink.view(np.uint32).astype(np.uint64).sum()) % 2 ** 32 == int(words.astype(np.uint64).sum()) % 2 ** 32
    # mode 1 stores nothing unless a wave total hits the fixed value
    marker = torch.full(sink.shape, 7, dtype=torch.int32, device="cuda")
    after = host(bn.bitnet_probe_stream_read(dev(words.view(np.int32)), sink=marker, mode=1))
    assert np.count_nonzero(after != 7) <= np.count_nonzero(sink.view(np.uint32) == 0x9E3779B9)
