"""Pins the CPU oracle to facts that do not come from the oracle itself:
the printed i2_s code map (golden bytes), closed forms, brute force against a
dense integer matmul, invariants of the mathematics, and exact rational
arithmetic.  CPU only."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- #
# canonical i2_s pack / unpack
# --------------------------------------------------------------------------- #
def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "i2s_canonical_bytes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, assign, expect = [s.strip() for s in line.split("|")]
            rows.append((name, assign, expect))
    return rows


@pytest.mark.parametrize("name,assign,expect", _golden_rows())
def test_pack_golden_bytes(name, assign, expect):
    t = np.zeros((1, 128), np.int8)
    for tok in assign.split():
        k, v = tok.split("=")
        if k == "fill":
            t[:] = int(v)
        else:
            t[0, int(k)] = int(v)
    P = oracle.pack_i2s(t)
    for tok in expect.split():
        j, hx = tok.split("=")
        assert P[0, int(j)] == int(hx, 16), (name, j, hex(P[0, int(j)]))
    assert np.array_equal(oracle.unpack_i2s(P, 128), t)


def test_pack_exhaustive_quadruples():
    # every one of the 81 (t0,t1,t2,t3) quadruples placed at weights j, 32+j, 64+j, 96+j
    quads = np.array(np.meshgrid(*[[-1, 0, 1]] * 4, indexing="ij")).reshape(4, -1).T  # 81 x 4
    T = np.zeros((81, 128), np.int8)
    for r, qd in enumerate(quads):
        j = r % 32
        for g in range(4):
            T[r, 32 * g + j] = qd[g]
    P = oracle.pack_i2s(T)
    for r, qd in enumerate(quads):
        j = r % 32
        want = sum((int(qd[g]) + 1) << (6 - 2 * g) for g in range(4))
        assert P[r, j] == want
    assert np.array_equal(oracle.unpack_i2s(P, 128), T)


@pytest.mark.parametrize("N,K", [(2560, 2560), (13824, 2560), (20480, 3200), (2560, 6912), (16, 128)])
def test_pack_roundtrip_config_shapes(N, K):
    T = wl.ternary_uniform(wl.rng_for(7, N, K), N, K)
    P = oracle.pack_i2s(T)
    assert P.shape == (N, K // 4)
    assert np.array_equal(oracle.unpack_i2s(P, K), T)


def test_pack_rejects_non_ternary_and_code3():
    T = np.zeros((1, 128), np.int8)
    T[0, 5] = 2
    with pytest.raises(ValueError):
        oracle.pack_i2s(T)
    P = np.full((1, 32), 0x55, np.uint8)
    P[0, 3] = 0xFF  # code 3
    with pytest.raises(ValueError):
        oracle.unpack_i2s(P, 128)


# --------------------------------------------------------------------------- #
# activation quantisation
# --------------------------------------------------------------------------- #
def _acts(seed, M, K, t=False):
    r = wl.rng_for(11, seed, M, K)
    return wl.student_t_act(r, M, K) if t else wl.normal_act(r, M, K)


@pytest.mark.parametrize("M,K,t", [(1, 2560, False), (8, 2560, False), (3, 3200, True), (5, 6912, False)])
def test_quant_invariants(M, K, t):
    xb = _acts(M + K, M, K, t)
    x = wl.bf16_to_f32(xb)
    q, s = oracle.quant_act_bf16(xb)
    q2, s2 = oracle.quant_act_f32(x)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    for m in range(M):
        am = np.abs(x[m]).max()
        k0 = int(np.abs(x[m]).argmax())
        assert abs(int(q[m, k0])) == 127 and np.sign(q[m, k0]) == np.sign(x[m, k0])
        assert np.abs(q[m]).max() == 127
        # dequant factor is amax/127 in fp32 (division correctly rounded: exact rational check)
        assert Fraction(float(s[m])) == Fraction(float(np.float32(am) / np.float32(127)))
        assert abs(Fraction(float(s[m])) - Fraction(float(am)) / 127) <= Fraction(float(s[m])) * Fraction(1, 2 ** 24)
        # round-to-nearest reconstruction: |x - q*s| <= s/2 (up to fp32 rounding of the ratio)
        err = np.abs(x[m].astype(np.float64) - q[m].astype(np.float64) * float(s[m]))
        assert err.max() <= float(s[m]) * (0.5 + 1e-5)
        # monotone in x
        order = np.argsort(x[m], kind="stable")
        assert np.all(np.diff(q[m][order].astype(np.int32)) >= 0)
    # sign symmetry and power-of-two scale invariance
    qn, sn = oracle.quant_act_f32(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for j in (-3, 5):
        qj, sj = oracle.quant_act_f32(x * np.float32(2.0 ** j))
        assert np.array_equal(qj, q)
        assert np.array_equal(sj, (s * np.float32(2.0 ** j)).astype(np.float32))


def test_quant_special_cases():
    x = np.zeros((2, 256), np.float32)
    x[1, 7] = -3.5
    x[1, 9] = 1.75  # exactly half of amax -> 63.5 -> ties to even -> 64
    x[1, 11] = 3.5 / 254.0 * 1.0  # tiny
    q, s = oracle.quant_act_f32(x)
    assert np.all(q[0] == 0)
    assert s[0] == np.float32(np.float32(1e-5) / np.float32(127))
    assert q[1, 7] == -127
    inv = np.float32(127) / np.float32(3.5)
    assert q[1, 9] == int(np.rint(np.float32(1.75) * inv))
    assert int(np.rint(np.float32(1.75) * inv)) in (63, 64)


def test_quant_matches_numpy_fp32():
    # an independent evaluation with numpy's own fp32 division and rint
    xb = _acts(3, 4, 2560)
    x = wl.bf16_to_f32(xb)
    q, s = oracle.quant_act_bf16(xb)
    am = np.maximum(np.abs(x).max(axis=1), np.float32(1e-5)).astype(np.float32)
    inv = (np.float32(127) / am).astype(np.float32)
    qq = np.clip(np.rint((x * inv[:, None]).astype(np.float32)), -127, 127).astype(np.int8)
    assert np.array_equal(q, qq)
    assert np.array_equal(s, (am / np.float32(127)).astype(np.float32))


# --------------------------------------------------------------------------- #
# integer product
# --------------------------------------------------------------------------- #
def _brute(T, Q):
    return (Q.astype(np.int64) @ T.astype(np.int64).T)


@pytest.mark.parametrize("M", [1, 2, 5, 8])
@pytest.mark.parametrize("N,K", [(16, 128), (32, 256), (64, 384), (48, 640)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_product_brute_force_tiny(M, N, K, seed):
    c = wl.small_case(seed, M, N, K)
    q, s = oracle.quant_act_bf16(c.x_bits)
    r = oracle.w2a8(oracle.pack_i2s(c.T), c.S, q, s, N, K)
    want = _brute(c.T, q)
    assert np.array_equal(r["acc"].astype(np.int64), want)
    assert np.array_equal(oracle.acc_dense(c.T, q).astype(np.int64), want)


def test_product_brute_force_config_shape():
    c = wl.config2(M=8)
    T, S = oracle.ternarize_absmean(c.W)
    q, s = oracle.quant_act_bf16(c.x_bits)
    r = oracle.w2a8(oracle.pack_i2s(T), S, q, s, c.N, c.K)
    assert np.array_equal(r["acc"].astype(np.int64), _brute(T, q))


def test_product_invariants():
    M, N, K = 3, 32, 512
    c = wl.small_case(5, M, N, K)
    q, s = oracle.quant_act_bf16(c.x_bits)
    base = oracle.w2a8(oracle.pack_i2s(c.T), c.S, q, s, N, K)
    # zero weights
    z = oracle.w2a8(oracle.pack_i2s(np.zeros_like(c.T)), c.S, q, s, N, K)
    assert np.all(z["acc"] == 0) and np.all(z["y"] == 0)
    # all +1 row -> activation sum; one-hot row -> one activation
    T2 = c.T.copy()
    T2[3] = 1
    T2[4] = 0
    T2[4, 200] = 1
    r2 = oracle.w2a8(oracle.pack_i2s(T2), c.S, q, s, N, K)
    assert np.array_equal(r2["acc"][:, 3], q.astype(np.int32).sum(axis=1))
    assert np.array_equal(r2["acc"][:, 4], q[:, 200].astype(np.int32))
    # sign flip negates exactly
    rn = oracle.w2a8(oracle.pack_i2s(-c.T), c.S, q, s, N, K)
    assert np.array_equal(rn["acc"], -base["acc"]) and np.array_equal(rn["y"], -base["y"])
    # linearity when the sum stays ternary
    mask = wl.rng_for(9).random(c.T.shape) < 0.5
    T_a = np.where(mask, c.T, 0).astype(np.int8)
    T_b = np.where(mask, 0, c.T).astype(np.int8)
    ra = oracle.w2a8(oracle.pack_i2s(T_a), c.S, q, s, N, K)
    rb = oracle.w2a8(oracle.pack_i2s(T_b), c.S, q, s, N, K)
    assert np.array_equal(ra["acc"] + rb["acc"], base["acc"])
    # token independence (batch rows are independent)
    r1 = oracle.w2a8(oracle.pack_i2s(c.T), c.S, q[1:2], s[1:2], N, K)
    assert np.array_equal(r1["acc"][0], base["acc"][1]) and np.array_equal(r1["y"][0], base["y"][1])


# --------------------------------------------------------------------------- #
# scale epilogue
# --------------------------------------------------------------------------- #
def test_scale_unit_scales_exact():
    M, N, K = 4, 64, 1024
    c = wl.small_case(2, M, N, K, skind="ones")
    q, _ = oracle.quant_act_bf16(c.x_bits)
    ones = np.ones(M, np.float32)
    r = oracle.w2a8(oracle.pack_i2s(c.T), c.S, q, ones, N, K)
    assert np.array_equal(r["y"], r["acc"].astype(np.float32))


def test_scale_power_of_two_scaling():
    M, N, K = 2, 32, 768
    c = wl.small_case(3, M, N, K)
    q, s = oracle.quant_act_bf16(c.x_bits)
    P = oracle.pack_i2s(c.T)
    r = oracle.w2a8(P, c.S, q, s, N, K)
    r2 = oracle.w2a8(P, (c.S * 2).astype(np.float32), q, s, N, K)
    r3 = oracle.w2a8(P, c.S, q, (s * 4).astype(np.float32), N, K)
    assert np.array_equal(r2["y"], r["y"] * 2)
    assert np.array_equal(r3["y"], r["y"] * 4)


def test_scale_block_index_closed_form():
    # one nonzero weight per row, in a different block per row: y = s_a * S[n,b] * t * q[k]
    M, N, K = 2, 16, 1024
    B = K // 128
    rng = wl.rng_for(21)
    S = rng.uniform(0.5, 2.0, size=(N, B)).astype(np.float32)
    T = np.zeros((N, K), np.int8)
    ks = []
    for n in range(N):
        k = int(rng.integers(0, K))
        T[n, k] = 1 if n % 2 else -1
        ks.append(k)
    xb = wl.normal_act(rng, M, K)
    q, s = oracle.quant_act_bf16(xb)
    r = oracle.w2a8(oracle.pack_i2s(T), S, q, s, N, K)
    for m in range(M):
        for n in range(N):
            k = ks[n]
            exact = Fraction(float(s[m])) * Fraction(float(S[n, k // 128])) * int(T[n, k]) * int(q[m, k])
            assert abs(Fraction(r["y64"][m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)
            assert r["acc"][m, n] == int(T[n, k]) * int(q[m, k])


def test_scale_magnitude_bounds_value():
    c = wl.small_case(4, 4, 64, 1280)
    q, s = oracle.quant_act_bf16(c.x_bits)
    r = oracle.w2a8(oracle.pack_i2s(c.T), c.S, q, s, c.N, c.K)
    assert np.all(np.abs(r["y64"]) <= r["mag"] * (1 + 1e-12))
    assert np.array_equal(r["y"], r["y64"].astype(np.float32))


# The tolerance magnitude mag = s_a * sum_b |S[n,b] * A[m,n,b]| (one absolute
# value per 128-weight block: [P3] "What i2_s actually is", one float scale per
# block, so the block sum A is the unit the scale multiplies).  Every fp32 / bf16
# parity bound is 1e-5 * max(|y|, mag), so mag is pinned exactly, not only from
# below: a per-weight magnitude, a wrong factor or a dropped block fails here.
def _block_sums(T, Q):
    """A[m, n, b] = sum over block b of T[n, k] * Q[m, k]: a dense int64 product per block."""
    N, K = T.shape
    B = K // 128
    return np.einsum("nbk,mbk->mnb", T.astype(np.int64).reshape(N, B, 128),
                     Q.astype(np.int64).reshape(Q.shape[0], B, 128))


@pytest.mark.parametrize("M,N,K,seed", [(1, 16, 128, 1), (3, 48, 640, 2), (8, 64, 2560, 3)])
def test_mag_is_sum_of_block_magnitudes_exactly(M, N, K, seed):
    # unit scales and s_a = 1: mag = sum_b |A_b| exactly (integers below 2^53)
    c = wl.small_case(seed, M, N, K, skind="ones")
    q, _ = oracle.quant_act_bf16(c.x_bits)
    r = oracle.w2a8(oracle.pack_i2s(c.T), c.S, q, np.ones(M, np.float32), N, K)
    A = _block_sums(c.T, q)
    want = np.abs(A).sum(axis=2)
    assert np.array_equal(r["mag"], want.astype(np.float64))
    # the data exercise the difference between the candidate definitions
    per_weight = np.abs(q.astype(np.int64)) @ np.abs(c.T.astype(np.int64)).T
    assert np.all(per_weight >= want) and np.any(per_weight > want)
    if K > 128:
        assert np.any(want > np.abs(A.sum(axis=2)))  # blocks of opposite sign cancel in y, not in mag


def test_mag_with_scales_matches_exact_rational():
    M, N, K = 2, 32, 1280
    c = wl.small_case(7, M, N, K)
    q, s = oracle.quant_act_bf16(c.x_bits)
    r = oracle.w2a8(oracle.pack_i2s(c.T), c.S, q, s, N, K)
    A = _block_sums(c.T, q)
    B = K // 128
    for m in range(M):
        for n in range(0, N, 3):
            exact = Fraction(float(s[m])) * sum(abs(Fraction(float(c.S[n, b])) * int(A[m, n, b])) for b in range(B))
            assert abs(Fraction(r["mag"][m, n]) - exact) <= exact * Fraction(2 * B, 2 ** 53)


def test_mag_closed_forms():
    K, B = 512, 4
    rng = wl.rng_for(31)
    q = rng.integers(1, 128, size=(1, K)).astype(np.int8)  # positive activations
    S = rng.uniform(0.5, 2.0, size=(3, B)).astype(np.float32)
    T = np.zeros((3, K), np.int8)
    T[0, 300] = -1                  # one nonzero weight: mag = |y|
    T[1, :] = 1                     # every block positive: mag = y
    T[2, :128] = 1                  # block 0 positive, block 1 negative: mag = |t0| + |t1|
    T[2, 128:256] = -1
    s_a = np.array([0.75], np.float32)
    r = oracle.w2a8(oracle.pack_i2s(T), S, q, s_a, 3, K)
    assert r["mag"][0, 0] == abs(r["y64"][0, 0]) and r["y64"][0, 0] < 0
    assert r["mag"][0, 1] == r["y64"][0, 1] > 0
    A = _block_sums(T, q)[0]
    t0 = Fraction(float(S[2, 0])) * int(A[2, 0])
    t1 = Fraction(float(S[2, 1])) * int(A[2, 1])
    assert t0 > 0 > t1
    assert Fraction(r["mag"][0, 2]) == Fraction(3, 4) * (abs(t0) + abs(t1))
    assert Fraction(r["y64"][0, 2]) == Fraction(3, 4) * (t0 + t1)


# Ties of the activation quantiser (reading R6: round half to even).  With
# amax = 127 the factor 127/amax is exactly 1, with amax = 254 exactly 1/2, so
# half-integers and odd integers / 2 land exactly on ties; numpy's rint rounds
# half to even, round-half-away-from-zero differs at 62.5, -62.5, 0.5, ...
def _tie_tokens():
    half = np.arange(-126.5, 127.0, 1.0, dtype=np.float32)          # 254 exact ties at inv = 1
    t1 = np.concatenate([[127.0, 0.0], half]).astype(np.float32)   # amax 127
    odd = np.arange(-253.0, 254.0, 2.0, dtype=np.float32)           # 254 exact ties at inv = 1/2
    t2 = np.concatenate([[254.0, 0.0], odd]).astype(np.float32)    # amax 254
    return np.stack([t1, t2])


def _expect_half_even(x):
    inv = (np.float32(127) / np.abs(x).max(axis=1)).astype(np.float32)
    assert inv[0] == 1.0 and inv[1] == 0.5
    return np.rint(x.astype(np.float64) * inv[:, None].astype(np.float64)).astype(np.int8)


def _check_tie_codes(q, x):
    want = _expect_half_even(x)
    assert np.array_equal(q, want)
    row = list(x[0])
    for v, code in [(62.5, 62), (-62.5, -62), (63.5, 64), (0.5, 0), (-0.5, 0), (1.5, 2), (126.5, 126)]:
        assert q[0, row.index(np.float32(v))] == code, v
    row = list(x[1])
    for v, code in [(125.0, 62), (-125.0, -62), (127.0, 64), (1.0, 0), (253.0, 126)]:
        assert q[1, row.index(np.float32(v))] == code, v


def test_quant_ties_round_half_to_even():
    x = _tie_tokens()
    q, s = oracle.quant_act_f32(x)
    _check_tie_codes(q, x)
    assert s[0] == np.float32(1.0) and s[1] == np.float32(2.0)
    # the same ties from bf16 inputs (every value above is exact in bf16)
    xb = wl.bf16_bits(x)
    assert np.array_equal(wl.bf16_to_f32(xb), x)
    qb, sb = oracle.quant_act_bf16(xb)
    assert np.array_equal(qb, q) and np.array_equal(sb, s)


def test_fold_quant_ties_round_half_to_even():
    x = _tie_tokens()
    lo = np.floor(x).astype(np.float32)        # h = lo + hi rebuilds x exactly
    hi = (x - lo).astype(np.float32)
    q, s = oracle.fold_quant(np.concatenate([lo, hi], axis=1))
    _check_tie_codes(q, x)
    q2, _ = oracle.fold_quant(np.concatenate([hi, lo], axis=1))  # the sum is symmetric
    assert np.array_equal(q2, q)


def test_glu_quant_ties_round_half_to_even():
    x = _tie_tokens()
    ones = np.ones_like(x)
    q, s = oracle.glu_quant(np.concatenate([ones, x], axis=1))          # relu(1)^2 * up = up
    _check_tie_codes(q, x)
    q4, s4 = oracle.glu_quant(np.concatenate([2 * ones, x / 4], axis=1))  # 4 * (up / 4), exact
    _check_tie_codes(q4, x)
    assert np.array_equal(s4, s)


# --------------------------------------------------------------------------- #
# absmean ternarisation
# --------------------------------------------------------------------------- #
def test_ternarize_recovers_scaled_ternary():
    rng = wl.rng_for(31)
    N, K = 32, 512
    T = wl.ternary_uniform(rng, N, K)
    T[:, ::128] = 1  # at least one nonzero per block
    c = np.float32(0.0371)
    T2, S = oracle.ternarize_absmean(T.astype(np.float32) * c)
    assert np.array_equal(T2, T)
    nnz = np.abs(T.reshape(N, K // 128, 128)).sum(axis=2)
    exact = (Fraction(float(c)) * nnz.astype(object)) / 128
    for n in range(N):
        for b in range(K // 128):
            assert S[n, b] == np.float32(float(exact[n, b]))


def test_ternarize_gaussian_zero_fraction_and_symmetry():
    W = wl.normal_weights(wl.rng_for(32), 2048, 1280, 0.02)
    T, S = oracle.ternarize_absmean(W)
    # |W|/gamma < 1/2 with gamma ~ E|W| = sigma*sqrt(2/pi): P(|Z| < sqrt(2/pi)/2) = 0.3101
    zf = float((T == 0).mean())
    assert abs(zf - 0.3101) < 0.01, zf
    assert abs(float((T == 1).mean()) - float((T == -1).mean())) < 0.005
    Tn, Sn = oracle.ternarize_absmean(-W)
    assert np.array_equal(Tn, -T) and np.array_equal(Sn, S)
    # scale is the block mean of |W| (exact rational mean, rounded once)
    blk = np.abs(W[:4, :128].astype(np.float64))
    for n in range(4):
        exact = sum(Fraction(float(v)) for v in blk[n]) / 128
        assert abs(Fraction(float(S[n, 0])) - exact) <= exact * Fraction(1, 2 ** 24)


def test_ternarize_zero_block_and_threshold():
    W = np.zeros((2, 256), np.float32)
    W[1, 128:] = 1.0
    W[1, 130] = 0.49  # gamma = (127 + 0.49)/128 < 1 -> ratio 0.49/gamma < 0.5 -> 0
    T, S = oracle.ternarize_absmean(W)
    assert np.all(T[0] == 0) and np.all(S[0] == 0) and np.all(T[1, :128] == 0) and S[1, 0] == 0
    assert T[1, 130] == 0 and T[1, 129] == 1


# --------------------------------------------------------------------------- #
# bf16 rounding and the chain junction
# --------------------------------------------------------------------------- #
def test_bf16_rne_points():
    one = 1.0
    ulp = 2.0 ** -7  # bf16 ulp at 1
    vals = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 2 ** -20, -2.5, 65280.0],
                    np.float32)
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x477F]
    assert list(oracle.f32_to_bf16(vals)) == want


def test_fold_quant_closed_form():
    H = 256
    y = np.zeros((1, 2 * H), np.float32)
    y[0, 3] = 1.0
    y[0, H + 3] = 2.0  # h[3] = 3 = amax
    y[0, 10] = -1.5
    y[0, H + 10] = 0.0
    q, s = oracle.fold_quant(y)
    assert q[0, 3] == 127 and q[0, 10] == int(np.rint(np.float32(-1.5) * (np.float32(127) / np.float32(3))))
    assert s[0] == np.float32(np.float32(3.0) / np.float32(127))
    assert np.count_nonzero(q) == 2


# Squared-ReLU gated junction: h = relu(gate)^2 * up (gate = first half).
def test_glu_quant_unit_gate_is_plain_quant():
    # gate = 1 -> relu(1)^2 = 1 exactly, so h = up and the junction reduces to
    # the plain per-token quantiser (pinned above against numpy fp32)
    rng = np.random.default_rng(41)
    M, H = 3, 384
    up = rng.standard_normal((M, H)).astype(np.float32)
    y = np.concatenate([np.ones((M, H), np.float32), up], axis=1)
    q, s = oracle.glu_quant(y)
    q0, s0 = oracle.quant_act_f32(up)
    assert np.array_equal(q, q0) and np.array_equal(s, s0)
    # halves swapped would read relu(up)^2 * 1: different codes
    qs, _ = oracle.glu_quant(np.concatenate([up, np.ones((M, H), np.float32)], axis=1))
    assert not np.array_equal(qs, q0)


def test_glu_quant_integer_gates_exact_squares():
    # integer gates, unit up: h is exactly relu(k)^2 (small integers are exact in fp32)
    H = 128
    k = np.tile(np.arange(-5, 12, dtype=np.float32), 8)[:H]
    y = np.concatenate([k, np.ones(H, np.float32)])[None, :]
    h_exact = np.where(k > 0, k * k, 0).astype(np.float32)[None, :]
    q, s = oracle.glu_quant(y)
    q0, s0 = oracle.quant_act_f32(h_exact)
    assert np.array_equal(q, q0) and np.array_equal(s, s0)
    assert s[0] == np.float32(np.float32(121.0) / np.float32(127.0))  # amax = 11^2
    assert q[0, list(k).index(11.0)] == 127 and np.all(q[0, k <= 0] == 0)


def test_glu_quant_negative_gate_and_symmetries():
    rng = np.random.default_rng(42)
    M, H = 2, 256
    g = rng.standard_normal((M, H)).astype(np.float32)
    u = rng.standard_normal((M, H)).astype(np.float32)
    # gate <= 0 everywhere -> h = 0 -> q = 0, s_a = 1e-5/127
    q, s = oracle.glu_quant(np.concatenate([-np.abs(g), u], axis=1))
    assert not np.any(q) and np.all(s == np.float32(np.float32(1e-5) / np.float32(127)))
    q, s = oracle.glu_quant(np.concatenate([g, u], axis=1))
    # up -> -up negates the codes (relu applies to the gate only)
    qn, sn = oracle.glu_quant(np.concatenate([g, -u], axis=1))
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # gate x 2 scales h by 4, up x 2 by 2: codes unchanged, factors scale exactly
    q4, s4 = oracle.glu_quant(np.concatenate([2 * g, u], axis=1))
    assert np.array_equal(q4, q) and np.array_equal(s4, 4 * s)
    q2, s2 = oracle.glu_quant(np.concatenate([g, 2 * u], axis=1))
    assert np.array_equal(q2, q) and np.array_equal(s2, 2 * s)
    # a gate flipped negative zeroes exactly its own outputs
    g2 = g.copy()
    g2[:, :64] = -np.abs(g2[:, :64])
    qz, _ = oracle.glu_quant(np.concatenate([g2, u], axis=1))
    assert not np.any(qz[:, :64])


# --------------------------------------------------------------------------- #
# Scale granularity G: 64 (ARM block), 128 (x86 block), 0 (one scale)
# --------------------------------------------------------------------------- #
def test_pack_g64_closed_forms_and_placement():
    for t, byte in [(0, 0x55), (1, 0xAA), (-1, 0x00)]:
        assert np.all(oracle.pack_i2s_g(np.full((2, 128), t, np.int8), 64) == byte)
    # worked example in 16-wide groups: t[0]=+1, t[16]=-1, t[32]=0, t[48]=+1 -> byte 0 = 10 00 01 10
    T = np.zeros((1, 128), np.int8)
    T[0, [0, 16, 32, 48]] = [1, -1, 0, 1]
    P = oracle.pack_i2s_g(T, 64)
    assert P[0, 0] == 0x86 and np.all(P[0, 1:] == 0x55)
    # a single +1 at k lands in byte 16*(k // 64) + k % 16, at shift 6 - 2 * ((k % 64) // 16)
    for k in [0, 5, 17, 33, 63, 64, 79, 127]:
        T = np.zeros((1, 128), np.int8)
        T[0, k] = 1
        P = oracle.pack_i2s_g(T, 64)
        want = np.full(32, 0x55, np.uint8)
        sh = 6 - 2 * ((k % 64) // 16)
        want[16 * (k // 64) + k % 16] = (0x55 & ~(3 << sh)) | (2 << sh)
        assert np.array_equal(P[0], want), k


def test_pack_g64_exhaustive_roundtrip():
    quads = np.array(np.meshgrid(*[[-1, 0, 1]] * 4, indexing="ij")).reshape(4, -1).T  # 81 x 4
    T = np.zeros((81, 128), np.int8)
    for r, qd in enumerate(quads):
        for g in range(4):
            T[r, 16 * g + 3] = qd[g]
            T[r, 64 + 16 * g + 9] = -qd[g]
    assert np.array_equal(oracle.unpack_i2s_g(oracle.pack_i2s_g(T, 64), 128, 64), T)
    assert len(set(oracle.pack_i2s_g(T, 64)[:, 3].tolist())) == 81


def test_pack_g_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.pack_i2s_g(np.full((1, 128), 2, np.int8), 64)
    with pytest.raises(ValueError):
        oracle.pack_i2s_g(np.zeros((1, 128), np.int8), 32)
    with pytest.raises(ValueError):
        oracle.unpack_i2s_g(np.full((1, 32), 0xFF, np.uint8), 128, 64)


@pytest.mark.parametrize("G", [0, 64])
def test_ternarize_g_recovers_scaled_ternary(G):
    rng = np.random.default_rng(43 + G)
    N, K = 4, 256  # N*K = 1024, a power of two: the per-matrix mean is exact
    T = (rng.integers(0, 3, size=(N, K)) - 1).astype(np.int8)
    T[:, ::32] = 1  # every block has a nonzero
    c = np.float32(0.75)
    T2, S = oracle.ternarize_absmean_g(T.astype(np.float32) * c, G)
    assert np.array_equal(T2, T)
    if G == 0:
        assert S.shape == (1,) and S[0] == np.float32(0.75 * np.count_nonzero(T) / (N * K))
    else:
        nnz = np.count_nonzero(T.reshape(N, K // 64, 64), axis=2)
        assert np.array_equal(S, (0.75 * nnz / 64).astype(np.float32))
    Tn, Sn = oracle.ternarize_absmean_g(-T.astype(np.float32) * c, G)
    assert np.array_equal(Tn, -T) and np.array_equal(Sn, S)


@pytest.mark.parametrize("G", [0, 64])
def test_ternarize_g_gaussian_zero_fraction(G):
    W = wl.rng_for(44, G).normal(0, 0.02, size=(256, 1024)).astype(np.float32)
    T, S = oracle.ternarize_absmean_g(W, G)
    # as for 128-blocks: P(|Z| < sqrt(2/pi)/2) = 0.3101; shorter blocks add a little spread
    assert abs(float((T == 0).mean()) - 0.3101) < 0.012


@pytest.mark.parametrize("G", [0, 64])
@pytest.mark.parametrize("M,N,K,seed", [(1, 16, 128, 1), (3, 32, 256, 2), (8, 64, 384, 3)])
def test_w2a8_g_brute_force_and_unit_scales(G, M, N, K, seed):
    r = wl.rng_for(45, G, seed)
    T = (r.integers(0, 3, size=(N, K)) - 1).astype(np.int8)
    Q = r.integers(-127, 128, size=(M, K)).astype(np.int8)
    P = oracle.pack_i2s_g(T, G)
    ones = np.ones(oracle.scale_shape(N, K, G), np.float32)
    out = oracle.w2a8_g(P, ones, Q, np.ones(M, np.float32), N, K, G)
    brute = Q.astype(np.int64) @ T.astype(np.int64).T
    assert np.array_equal(out["acc"], brute)
    assert np.array_equal(out["y"], brute.astype(np.float32))  # |acc| < 2^24: exact


def test_w2a8_g64_uses_each_half_scale():
    # +1 weights only in one 64-half of a 128-block, unit activations: y = s_a * S[half] * 64
    N, K = 16, 256
    S = wl.rng_for(46).uniform(0.5, 2, size=(N, K // 64)).astype(np.float32)
    Q = np.ones((1, K), np.int8)
    s_a = np.array([0.5], np.float32)
    for half in range(4):
        T = np.zeros((N, K), np.int8)
        T[:, 64 * half:64 * half + 64] = 1
        out = oracle.w2a8_g(oracle.pack_i2s_g(T, 64), S, Q, s_a, N, K, 64)
        assert np.array_equal(out["acc"][0], np.full(N, 64))
        assert np.array_equal(out["y64"][0], 0.5 * S[:, half].astype(np.float64) * 64)


def test_w2a8_g_reduces_to_block128():
    # exact reductions to the pinned 128-block product (scales from {0.5, 1, 1.5, 2}:
    # every partial sum is exact in fp64, so the results agree bit for bit)
    r = wl.rng_for(47)
    M, N, K = 4, 48, 384
    T = (r.integers(0, 3, size=(N, K)) - 1).astype(np.int8)
    Q = r.integers(-127, 128, size=(M, K)).astype(np.int8)
    s_a = r.uniform(0.01, 0.1, size=M).astype(np.float32)
    S128 = (r.integers(1, 5, size=(N, K // 128)) * 0.5).astype(np.float32)
    ref = oracle.w2a8(oracle.pack_i2s(T), S128, Q, s_a, N, K)
    out64 = oracle.w2a8_g(oracle.pack_i2s_g(T, 64), np.repeat(S128, 2, axis=1), Q, s_a, N, K, 64)
    assert np.array_equal(out64["y64"], ref["y64"]) and np.array_equal(out64["acc"], ref["acc"])
    c = np.float32(1.5)
    ref_c = oracle.w2a8(oracle.pack_i2s(T), np.full((N, K // 128), c, np.float32), Q, s_a, N, K)
    out0 = oracle.w2a8_g(oracle.pack_i2s_g(T, 0), np.array([c]), Q, s_a, N, K, 0)
    assert np.array_equal(out0["y64"], ref_c["y64"]) and np.array_equal(out0["y"], ref_c["y"])
    # sign flip negates; doubling the one scale doubles y exactly
    neg = oracle.w2a8_g(oracle.pack_i2s_g(-T, 0), np.array([c]), Q, s_a, N, K, 0)
    assert np.array_equal(neg["y64"], -out0["y64"])
    dbl = oracle.w2a8_g(oracle.pack_i2s_g(T, 0), np.array([2 * c]), Q, s_a, N, K, 0)
    assert np.array_equal(dbl["y64"], 2 * out0["y64"])
