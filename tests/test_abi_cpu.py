"""CPU-only checks of the C ABI library: it loads, exports every symbol the
header declares, its host-side offline code (ternarise / pack / repack /
unpack) agrees with the oracle bit for bit, the tile layout matches the
header's specification, and invalid calls are rejected before any HIP call
(no kernel is launched here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_gemv_i2_amd as bn
import oracle
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(bitnet_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    syms = _declared_symbols()
    assert len(syms) >= 13
    lib = bn.lib()
    for s in syms:
        assert hasattr(lib, s), s


def test_one_hip_runtime_whatever_the_import_order():
    """The library shares torch's HIP runtime even when it is loaded before torch
    is imported (two runtimes in one process would own different memory and
    streams).  Runs in fresh interpreters; no GPU call is made."""
    import ast
    import subprocess
    import sys

    pytest.importorskip("torch")
    maps = "sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l})"
    for first in ("import bit_gemv_i2_amd as bn; bn.lib(); import torch",
                  "import torch; import bit_gemv_i2_amd as bn; bn.lib()"):
        out = subprocess.run([sys.executable, "-c", f"{first}; print({maps})"], cwd=ROOT,
                             capture_output=True, text=True, timeout=300)
        assert out.returncode == 0, out.stderr
        runtimes = ast.literal_eval(out.stdout.strip().splitlines()[-1])
        assert len(runtimes) == 1, (first, runtimes)


def test_status_strings():
    assert bn.bitnet_status_str(0) == "ok"
    assert "invalid" in bn.bitnet_status_str(1)
    assert "shape" in bn.bitnet_status_str(2)
    assert "HIP" in bn.bitnet_status_str(3)
    assert bn.bitnet_status_str(99) == "unknown status"


@pytest.mark.parametrize("N,K,ok", [(2560, 2560, True), (13824, 2560, True), (20480, 3200, True), (2560, 6912, True),
                                    (16, 128, True), (8, 128, False), (2560, 2500, False), (24, 128, False),
                                    (0, 128, False), (16, 0, False), (-16, 128, False)])
def test_shape_rules_and_sizes(N, K, ok):
    assert (bn.bitnet_check_shape(N, K) == bn.BITNET_OK) == ok
    assert bn.bitnet_packed_bytes(N, K) == (N * K // 4 if ok else 0)
    assert bn.bitnet_scale_count(N, K) == (N * K // 128 if ok else 0)


# ------------------------------------------------------------------ decode split-K geometry (host logic)
MI355X_CUS, MI355X_SLOTS = 256, 256 * 32  # 256 CUs x 2048 threads / 64


# waves x blocks per wave on a 256-CU device, as measured best (at most one 16-row workgroup
# per CU: busiest SIMD ceil(waves/4) x blocks; more workgroups than fit: blocks grow until
# every workgroup is resident; otherwise about 4 blocks per wave)
@pytest.mark.parametrize("N,K,want", [(2560, 2560, (4, 5)), (2560, 3200, (4, 7)), (2560, 6912, (8, 7)),
                                      (2560, 1280, (4, 3)), (4096, 2560, (4, 5)), (2560, 4096, (8, 4)),
                                      (4096, 1664, (4, 4)), (2560, 384, (1, 3)), (13824, 2560, (5, 4)),
                                      (20480, 3200, (5, 5)), (6912, 2560, (5, 4)), (2560, 12416, (11, 9))])
def test_gemv_split_on_a_256_cu_device(N, K, want):
    assert bn.bitnet_gemv_split(N, K, MI355X_CUS, MI355X_SLOTS) == want


@pytest.mark.parametrize("N,K,want", [(2560, 2560, (5, 4)), (20480, 3200, (7, 4)), (2560, 6912, (11, 5)),
                                      (16, 128, (1, 1)), (16, 12288, (12, 8))])
def test_gemv_split_without_device_information_is_the_base_split(N, K, want):
    assert bn.bitnet_gemv_split(N, K) == want


def _busiest_simd(w, p):
    return -(-w // 4) * p


@pytest.mark.parametrize("cus", [0, 32, 80, 256, 304])
def test_gemv_split_invariants(cus):
    slots = cus * 32
    for K in range(128, 12416 + 1, 128 * 3):
        nblk = K // 128
        base_w, base_p = bn.bitnet_gemv_split(16, K)
        for N in (16, 1024, 2560, 4096, 8192, 13824, 20480, 40960):
            w, p = bn.bitnet_gemv_split(N, K, cus, slots)
            assert 1 <= w <= 12 and p >= 1
            assert (w - 1) * p < nblk <= w * p, (N, K, w, p)  # every block covered, no idle wave
            if base_p <= 8:
                assert p <= 8, (N, K, w, p)  # fused forms stay available
            wgs = N // 16
            if cus and wgs <= cus and nblk >= 8 and base_p <= 8:
                # no split within the limits has a less loaded SIMD
                best = min(_busiest_simd(-(-nblk // q), q) for q in range(1, min(8, nblk) + 1)
                           if -(-nblk // q) <= 12)
                assert _busiest_simd(w, p) == best, (N, K, w, p, best)
            if cus and wgs > cus and p < min(8, nblk):
                assert wgs * w <= slots, (N, K, w, p)  # the whole grid is resident
            if not cus:
                assert (w, p) == (base_w, base_p)


def test_gemv_split_rejects_bad_arguments():
    for N, K in [(8, 128), (2560, 2500)]:
        with pytest.raises(bn.BitnetError) as ei:
            bn.bitnet_gemv_split(N, K, MI355X_CUS, MI355X_SLOTS)
        assert ei.value.status == bn.BITNET_ERR_UNSUPPORTED_SHAPE
    with pytest.raises(bn.BitnetError) as ei:
        bn.bitnet_gemv_split(2560, 2560, -1, MI355X_SLOTS)
    assert ei.value.status == bn.BITNET_ERR_INVALID_ARG
    w = ctypes.c_int(0)
    assert bn.lib().bitnet_gemv_split(2560, 2560, 0, 0, None, ctypes.byref(w)) == bn.BITNET_ERR_INVALID_ARG


# ------------------------------------------------------------------ host offline code vs oracle
@pytest.mark.parametrize("seed,N,K", [(0, 16, 128), (1, 48, 384), (2, 2560, 2560), (3, 13824, 2560)])
def test_ternarize_matches_oracle(seed, N, K):
    W = wl.normal_weights(wl.rng_for(41, seed), N, K, 0.02)
    W[0, :128] = 0.0  # a zero block
    t_lib, s_lib = bn.bitnet_ternarize_absmean(W)
    t_or, s_or = oracle.ternarize_absmean(W)
    assert np.array_equal(t_lib, t_or)
    assert np.array_equal(s_lib.view(np.uint32), s_or.view(np.uint32))


def test_ternarize_config2_matches_oracle():
    c = wl.config2()
    t_lib, s_lib = bn.bitnet_ternarize_absmean(c.W)
    t_or, s_or = oracle.ternarize_absmean(c.W)
    assert np.array_equal(t_lib, t_or) and np.array_equal(s_lib, s_or)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 640), (2560, 2560), (2560, 6912), (20480, 3200)])
def test_pack_unpack_roundtrip_and_repack_from_canonical(N, K):
    r = wl.rng_for(43, N, K)
    T = wl.ternary_uniform(r, N, K)
    S = wl.uniform_scales(r, N, K)
    packed, st = bn.bitnet_pack_i2s(T, S)
    assert packed.size == N * K // 4 and st.size == N * K // 128
    T2, S2 = bn.bitnet_unpack_i2s(packed, st, N, K)
    assert np.array_equal(T2, T) and np.array_equal(S2, S)
    # the oracle's canonical i2_s bytes repack to the identical tile buffer
    packed2, st2 = bn.bitnet_repack_i2s(oracle.pack_i2s(T), S, K)
    assert np.array_equal(packed2, packed) and np.array_equal(st2, st)


def test_tile_layout_matches_header_spec():
    # place single weights and check the byte/bit position the header specifies
    N, K = 32, 256
    nblk = K // 128
    for (n, k, t) in [(0, 0, 1), (17, 130, -1), (31, 255, 1), (5, 64 + 16 * 3 + 4 * 2 + 1, -1), (16, 7, 1)]:
        T = np.zeros((N, K), np.int8)
        T[n, k] = t
        packed, _ = bn.bitnet_pack_i2s(T, np.ones((N, nblk), np.float32))
        Tt, j = divmod(n, 16)
        b, r = divmod(k, 128)
        s, r = divmod(r, 64)
        g, e = divmod(r, 16)
        i, p = divmod(e, 4)
        byte = (Tt * nblk + b) * 512 + (16 * g + j) * 8 + 4 * s + p
        want = np.zeros_like(packed)
        want[byte] = (t & 3) << (2 * i)
        assert np.array_equal(packed, want), (n, k)
    # scales: row 16T+j, block b at (T*nblk + b)*16 + j
    S = np.arange(N * nblk, dtype=np.float32).reshape(N, nblk)
    _, st = bn.bitnet_pack_i2s(np.zeros((N, K), np.int8), S)
    for n in range(N):
        for b in range(nblk):
            assert st[((n // 16) * nblk + b) * 16 + n % 16] == S[n, b]


def test_pack_rejects_bad_input_without_writing():
    T = np.zeros((16, 128), np.int8)
    T[3, 3] = 2
    with pytest.raises(bn.BitnetError) as ei:
        bn.bitnet_pack_i2s(T, np.ones((16, 1), np.float32))
    assert ei.value.status == bn.BITNET_ERR_INVALID_ARG
    P = np.full((16, 32), 0x55, np.uint8)
    P[2, 2] = 0xC0 | 0x15  # code 3 in group 0
    with pytest.raises(bn.BitnetError):
        bn.bitnet_repack_i2s(P, np.ones((16, 1), np.float32), 128)
    with pytest.raises(bn.BitnetError) as ei:
        bn.bitnet_pack_i2s(np.zeros((24, 128), np.int8), np.ones((24, 1), np.float32))


# ------------------------------------------------------------------ validation before any HIP call
_FAKE = ctypes.c_void_p(0x100000)       # aligned, non-null, never dereferenced
_MIS = ctypes.c_void_p(0x100004)        # misaligned
_NULL = ctypes.c_void_p(0)


@pytest.mark.parametrize("M,N,K,ptr,want", [
    (0, 2560, 2560, _FAKE, bn.BITNET_ERR_UNSUPPORTED_SHAPE),
    (17, 2560, 2560, _FAKE, bn.BITNET_ERR_UNSUPPORTED_SHAPE),
    (1, 2560, 2500, _FAKE, bn.BITNET_ERR_UNSUPPORTED_SHAPE),
    (1, 2568, 2560, _FAKE, bn.BITNET_ERR_UNSUPPORTED_SHAPE),
    (1, 2560, 2560, _NULL, bn.BITNET_ERR_INVALID_ARG),
    (1, 2560, 2560, _MIS, bn.BITNET_ERR_INVALID_ARG),
])
def test_gemv_validation(M, N, K, ptr, want):
    st = bn.lib().bitnet_w2a8_gemv(ptr, _FAKE, _FAKE, _FAKE, _FAKE, M, N, K, _NULL)
    assert st == want


def test_decode_outputs_must_be_16_byte_aligned():
    # the decode kernels store each token's four consecutive rows as one 16-byte piece
    L = bn.lib()
    assert L.bitnet_w2a8_gemv(_FAKE, _FAKE, _FAKE, _FAKE, _MIS, 8, 2560, 2560, _NULL) == bn.BITNET_ERR_INVALID_ARG
    assert L.bitnet_w2a8_gemv_g(_FAKE, _FAKE, _FAKE, _FAKE, _MIS, 8, 2560, 2560, 0, _NULL) == \
        bn.BITNET_ERR_INVALID_ARG
    assert L.bitnet_w2a8_gemv_act(_FAKE, _FAKE, _FAKE, 0, _MIS, _NULL, _NULL, 1, 2560, 2560, _NULL) == \
        bn.BITNET_ERR_INVALID_ARG
    assert L.bitnet_w2a8_acc_i32(_FAKE, _FAKE, _MIS, 8, 2560, 2560, _NULL) == bn.BITNET_ERR_INVALID_ARG


def test_gemm_acc_quant_validation():
    L = bn.lib()
    assert L.bitnet_w2a8_gemm(_FAKE, _FAKE, _FAKE, _FAKE, _FAKE, 7, 4, 16, 128, _NULL) == bn.BITNET_ERR_INVALID_ARG
    assert L.bitnet_w2a8_gemm(_FAKE, _FAKE, _FAKE, _FAKE, _FAKE, 0, 0, 16, 128, _NULL) == \
        bn.BITNET_ERR_UNSUPPORTED_SHAPE
    assert L.bitnet_w2a8_gemm(_FAKE, _FAKE, _MIS, _FAKE, _FAKE, 0, 4, 16, 128, _NULL) == bn.BITNET_ERR_INVALID_ARG
    assert L.bitnet_w2a8_acc_i32(_FAKE, _FAKE, _FAKE, 4, 16, 100, _NULL) == bn.BITNET_ERR_UNSUPPORTED_SHAPE
    assert L.bitnet_w2a8_acc_i32(_FAKE, _FAKE, _NULL, 4, 16, 128, _NULL) == bn.BITNET_ERR_INVALID_ARG
    assert L.bitnet_quant_act(_FAKE, 5, 1, 256, _FAKE, _FAKE, _NULL) == bn.BITNET_ERR_INVALID_ARG
    assert L.bitnet_quant_act(_FAKE, 0, 1, 250, _FAKE, _FAKE, _NULL) == bn.BITNET_ERR_UNSUPPORTED_SHAPE
    assert L.bitnet_quant_act(_FAKE, 0, 0, 256, _FAKE, _FAKE, _NULL) == bn.BITNET_ERR_UNSUPPORTED_SHAPE
    assert L.bitnet_quant_act(_MIS, 0, 1, 256, _FAKE, _FAKE, _NULL) == bn.BITNET_ERR_INVALID_ARG
    assert L.bitnet_quant_act_fold(_FAKE, 1, 24, _FAKE, _FAKE, _NULL) == bn.BITNET_ERR_UNSUPPORTED_SHAPE
    assert L.bitnet_quant_act_fold(_NULL, 1, 32, _FAKE, _FAKE, _NULL) == bn.BITNET_ERR_INVALID_ARG


def test_lut_gemv_validation():
    L = bn.lib()
    f = L.bitnet_w2a8_gemv_lut
    assert f(_NULL, _FAKE, _FAKE, _FAKE, _FAKE, _NULL, 2560, 2560, 0, _NULL) == bn.BITNET_ERR_INVALID_ARG
    assert f(_FAKE, _FAKE, _FAKE, _FAKE, _NULL, _FAKE, 2560, 2560, 0, _NULL) == bn.BITNET_ERR_INVALID_ARG
    assert f(_MIS, _FAKE, _FAKE, _FAKE, _FAKE, _NULL, 2560, 2560, 0, _NULL) == bn.BITNET_ERR_INVALID_ARG
    assert f(_FAKE, _FAKE, _FAKE, _FAKE, _FAKE, ctypes.c_void_p(0x100002), 2560, 2560, 1, _NULL) == \
        bn.BITNET_ERR_INVALID_ARG
    for tiles in (3, 8, -1):
        assert f(_FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _NULL, 2560, 2560, tiles, _NULL) == bn.BITNET_ERR_INVALID_ARG
    assert f(_FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _NULL, 2560, 2500, 0, _NULL) == bn.BITNET_ERR_UNSUPPORTED_SHAPE
    assert f(_FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _NULL, 2568, 2560, 0, _NULL) == bn.BITNET_ERR_UNSUPPORTED_SHAPE
    assert f(_FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _NULL, 16, (1 << 22) + 128, 0, _NULL) == \
        bn.BITNET_ERR_UNSUPPORTED_SHAPE


def test_product_path_has_no_fallback(monkeypatch):
    # a missing library must raise, never compute on the CPU
    monkeypatch.setattr(bn, "_lib", None)
    monkeypatch.setattr(bn, "LIB_PATH", os.path.join(ROOT, "does_not_exist.so"))
    with pytest.raises(RuntimeError):
        bn.lib()


def test_junction_codes():
    assert [bn.junction_code(j) for j in (False, None, "none", 0)] == [0, 0, 0, 0]
    assert [bn.junction_code(j) for j in (True, "sum", 1)] == [1, 1, 1]
    assert [bn.junction_code(j) for j in ("relu2_glu", 2)] == [2, 2]
    for bad in ("relu", 3, -1, 2.5):
        with pytest.raises(ValueError):
            bn.junction_code(bad)


# ------------------------------------------------------------------ scale granularity (host side)
@pytest.mark.parametrize("G", [0, 64])
@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (272, 2560)])
def test_ternarize_g_matches_oracle(G, N, K):
    W = wl.rng_for(91, G, N, K).normal(0, 0.02, size=(N, K)).astype(np.float32)
    T, S = bn.bitnet_ternarize_absmean_g(W, G)
    To, So = oracle.ternarize_absmean_g(W, G)
    assert np.array_equal(T, To) and np.array_equal(S, So)


def test_ternarize_g0_config2_shape_matches_oracle():
    # one gamma over 35 M weights: the fp64 sum runs in the same row-major order on both sides
    W = wl.rng_for(92).normal(0, 0.02, size=(13824, 2560)).astype(np.float32)
    T, S = bn.bitnet_ternarize_absmean_g(W, 0)
    To, So = oracle.ternarize_absmean_g(W, 0)
    assert S[0] == So[0] and np.array_equal(T, To)


@pytest.mark.parametrize("G", [0, 64, 128])
@pytest.mark.parametrize("N,K", [(16, 128), (80, 640), (2560, 2560)])
def test_pack_g_roundtrip_and_repack_from_canonical(G, N, K):
    r = wl.rng_for(93, G, N, K)
    T = wl.ternary_uniform(r, N, K)
    S = r.uniform(0.5, 2, size=oracle.scale_shape(N, K, G)).astype(np.float32)
    p, st = bn.bitnet_pack_i2s_g(T, S, G)
    assert st.size == bn.bitnet_scale_count_g(N, K, G) == (1 if G == 0 else N * K // G)
    T2, S2 = bn.bitnet_unpack_i2s_g(p, st, N, K, G)
    assert np.array_equal(T2, T) and np.array_equal(S2, S)
    # the packed weights do not depend on the scale granularity
    assert np.array_equal(p, bn.bitnet_pack_i2s(T, np.ones((N, K // 128), np.float32))[0])
    p3, st3 = bn.bitnet_repack_i2s_g(oracle.pack_i2s_g(T, G), S, K, G)
    assert np.array_equal(p3, p) and np.array_equal(st3, st)


def test_tiled_scale_order_g64():
    # [tile][128-block][16 rows][2 halves]: the scale of row n, 64-block c sits at
    # (((n // 16) * (K // 128) + c // 2) * 16 + n % 16) * 2 + c % 2
    N, K = 32, 384
    S = np.arange(N * K // 64, dtype=np.float32).reshape(N, K // 64)
    _, st = bn.bitnet_pack_i2s_g(np.zeros((N, K), np.int8), S, 64)
    for n in range(N):
        for c in range(K // 64):
            assert st[(((n // 16) * (K // 128) + c // 2) * 16 + n % 16) * 2 + c % 2] == S[n, c]


def test_g_variants_reject_bad_scale_block():
    T = np.zeros((16, 128), np.int8)
    assert bn.bitnet_scale_count_g(16, 128, 32) == 0
    st = bn.lib().bitnet_pack_i2s_g(T.ctypes.data, np.ones(4, np.float32).ctypes.data, 16, 128, 32,
                                    np.empty(512, np.uint8).ctypes.data, np.empty(64, np.float32).ctypes.data)
    assert st == bn.BITNET_ERR_INVALID_ARG
    for sb in (32, 96, -1):
        assert bn.lib().bitnet_w2a8_gemv_g(None, None, None, None, None, 1, 16, 128, sb, None) == \
            bn.BITNET_ERR_INVALID_ARG
        assert bn.lib().bitnet_w2a8_gemm_g(None, None, None, None, None, 0, 1, 16, 128, sb, None) == \
            bn.BITNET_ERR_INVALID_ARG


# Every device wrapper checks its tensors against the library's size authorities
# (bitnet_packed_bytes, bitnet_scale_count[_g], M*K, M*N) before it takes a pointer:
# a mis-sized buffer raises here, on host tensors, long before any launch could read or
# write past it ([P4] "Matrix memory bounds and stride safety").
def _operands(torch, M=2, N=48, K=384, G=128):
    ns = bn.bitnet_scale_count(N, K) if G == 128 else bn.bitnet_scale_count_g(N, K, G)
    return dict(packed=torch.zeros(bn.bitnet_packed_bytes(N, K), dtype=torch.uint8),
                scales=torch.zeros(ns, dtype=torch.float32),
                q=torch.zeros((M, K), dtype=torch.int8), s_a=torch.zeros(M, dtype=torch.float32),
                y=torch.zeros((M, N), dtype=torch.float32), M=M, N=N, K=K)


def _calls(torch, o):
    N, K = o["N"], o["K"]
    return {
        "gemv": lambda **k: bn.bitnet_w2a8_gemv(k["packed"], k["scales"], k["q"], k["s_a"], N, K, y=k["y"]),
        "gemm": lambda **k: bn.bitnet_w2a8_gemm(k["packed"], k["scales"], k["q"], k["s_a"], N, K, y=k["y"]),
        "gemv_g": lambda **k: bn.bitnet_w2a8_gemv_g(k["packed"], k["scales"], k["q"], k["s_a"], N, K, 128, y=k["y"]),
        "gemm_g": lambda **k: bn.bitnet_w2a8_gemm_g(k["packed"], k["scales"], k["q"], k["s_a"], N, K, 128, y=k["y"]),
        "acc": lambda **k: bn.bitnet_w2a8_acc_i32(k["packed"], k["q"], N, K,
                                                   acc=torch.zeros((k["q"].shape[0], N), dtype=torch.int32)),
    }


@pytest.mark.parametrize("which", ["gemv", "gemm", "gemv_g", "gemm_g", "acc"])
def test_wrappers_reject_mis_sized_operands_before_any_launch(which):
    torch = pytest.importorskip("torch")
    o = _operands(torch)
    call = _calls(torch, o)[which]
    args = {k: o[k] for k in ("packed", "scales", "q", "s_a", "y")}
    # correct sizes pass every check and stop only at the device test
    with pytest.raises(ValueError, match="device tensor"):
        call(**args)
    bad = {
        "packed": torch.zeros(o["packed"].numel() - 16, dtype=torch.uint8),
        "scales": torch.zeros(o["scales"].numel() + 1, dtype=torch.float32),
        "q": torch.zeros((o["M"], o["K"] - 128), dtype=torch.int8),
        "s_a": torch.zeros(o["M"] + 1, dtype=torch.float32),
        "y": torch.zeros((o["M"], o["N"] - 16), dtype=torch.float32),
    }
    wrong_dtype = {"packed": torch.zeros(o["packed"].numel(), dtype=torch.int8),
                   "q": torch.zeros((o["M"], o["K"]), dtype=torch.uint8),
                   "y": torch.zeros((o["M"], o["N"]), dtype=torch.float64)}
    for name, t in list(bad.items()) + list(wrong_dtype.items()):
        if which == "acc" and name in ("scales", "s_a", "y"):
            continue
        with pytest.raises(ValueError, match=name if name != "q" else "q"):
            call(**dict(args, **{name: t}))
    if which == "acc":
        with pytest.raises(ValueError, match="acc"):
            bn.bitnet_w2a8_acc_i32(o["packed"], o["q"], o["N"], o["K"],
                                   acc=torch.zeros((o["M"], o["N"] + 16), dtype=torch.int32))


def test_wrappers_reject_unsupported_weight_shapes_and_formats():
    torch = pytest.importorskip("torch")
    o = _operands(torch)
    with pytest.raises(bn.BitnetError) as ei:    # N not a multiple of 16
        bn.bitnet_w2a8_gemv(o["packed"], o["scales"], o["q"], o["s_a"], 40, o["K"])
    assert ei.value.status == bn.BITNET_ERR_UNSUPPORTED_SHAPE
    with pytest.raises(bn.BitnetError) as ei:    # no such scale granularity
        bn.bitnet_w2a8_gemv_g(o["packed"], o["scales"], o["q"], o["s_a"], o["N"], o["K"], 32)
    assert ei.value.status == bn.BITNET_ERR_INVALID_ARG
    # a scale buffer of the 128 format handed to the 64 format is too small
    with pytest.raises(ValueError, match="scales"):
        bn.bitnet_w2a8_gemv_g(o["packed"], o["scales"], o["q"], o["s_a"], o["N"], o["K"], 64)


def test_other_wrappers_check_their_outputs():
    torch = pytest.importorskip("torch")
    x = torch.zeros((3, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q"):
        bn.bitnet_quant_act(x, q=torch.zeros((3, 128), dtype=torch.int8))
    with pytest.raises(ValueError, match="s_a"):
        bn.bitnet_quant_act(x, s_a=torch.zeros(2, dtype=torch.float32))
    y2 = torch.zeros((3, 512), dtype=torch.float32)
    with pytest.raises(ValueError, match="q"):
        bn.bitnet_quant_act_fold(y2, q=torch.zeros((3, 512), dtype=torch.int8))
    with pytest.raises(ValueError, match="s_a"):
        bn.bitnet_quant_act_relu2_glu(y2, s_a=torch.zeros(4, dtype=torch.float32))
    o = _operands(torch, M=1)
    xb = torch.zeros((1, o["K"]), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q_out"):
        bn.bitnet_w2a8_gemv_act(o["packed"], o["scales"], xb, o["N"], o["K"],
                                q_out=torch.zeros((1, o["K"] // 2), dtype=torch.int8))
    with pytest.raises(ValueError, match="y"):
        bn.bitnet_w2a8_gemv_act(o["packed"], o["scales"], xb, o["N"], o["K"],
                                y=torch.zeros((1, o["N"] + 16), dtype=torch.float32))
    with pytest.raises(ValueError, match="acc"):
        bn.bitnet_w2a8_gemv_lut(o["packed"], o["scales"], o["q"], o["s_a"], o["N"], o["K"],
                                acc=torch.zeros((1, 16), dtype=torch.int32))
    with pytest.raises(ValueError, match="sink"):
        bn.bitnet_probe_stream_read(torch.zeros(4096, dtype=torch.uint8), sink=torch.zeros(0, dtype=torch.int32))


# The one-launch (persistent) chain: its host-side plan chooses, per layer, the row tiles
# per workgroup (4, 2 or 1: as few workgroups as fit), the waves per tile and blocks per
# wave, and lays out one output buffer per layer after a 256-byte status block.
def _plan(shapes, folds, M=1, xdt=0, cus=256):
    n = len(shapes)
    arr = (bn.ChainLayer * n)()
    for i, ((N, K), f) in enumerate(zip(shapes, folds)):
        arr[i] = bn.ChainLayer(0x100000, 0x200000, N, K, f)
    nb = bn.lib().bitnet_w2a8_persist_table_bytes(n)
    host = np.zeros(nb, np.uint8)
    ws = ctypes.c_size_t(0)
    st = bn.lib().bitnet_w2a8_persist_prepare(ctypes.cast(arr, ctypes.c_void_p), n, M, xdt, cus,
                                               host.ctypes.data_as(ctypes.c_void_p), nb, ctypes.byref(ws))
    return st, host.view(np.int32).reshape(n, 16), ws.value


def test_persistent_plan_of_the_stack_layers():
    shapes = [(2560, 2560)] * 4 + [(13824, 2560), (2560, 6912)]
    folds = [0, 0, 0, 0, 0, 1]
    st, t, ws = _plan(shapes, folds)
    assert st == bn.BITNET_OK
    assert bn.lib().bitnet_w2a8_persist_table_bytes(6) == 6 * 64
    # int32 fields after the pointers and offsets: N, K, xm, tp, nw, per, nwg
    fields = [tuple(row[8:15]) for row in t]
    assert fields[0] == (2560, 2560, 0, 4, 4, 5, 40)       # bf16 input, 4 tiles x (4 waves x 5 blocks)
    assert fields[1] == (2560, 2560, 4, 4, 4, 5, 40)       # previous output
    assert fields[4] == (13824, 2560, 4, 4, 4, 5, 216)     # 864 tiles on 216 workgroups
    assert fields[5] == (2560, 6912, 5, 2, 8, 7, 80)       # folded input: 2 tiles x (8 waves x 7 blocks)
    offs = t.view(np.int64).reshape(6, 8)
    assert list(offs[:, 2]) == [-1, 256, 256 + 10240, 256 + 20480, 256 + 30720, 256 + 40960]  # inputs
    assert list(offs[:, 3]) == [256, 256 + 10240, 256 + 20480, 256 + 30720, 256 + 40960, -1]   # outputs
    assert ws == 256 + 4 * 10240 + 55296
    # the squared-ReLU gate is its own input form
    _, t2, _ = _plan(shapes, [0, 0, 0, 0, 0, 2])
    assert t2[5][10] == 6


def test_persistent_plan_rejections():
    ok = [(256, 512), (384, 256)]
    assert _plan(ok, [0, 0])[0] == bn.BITNET_OK
    assert _plan(ok, [0, 0], M=2)[0] == bn.BITNET_ERR_UNSUPPORTED_SHAPE      # batch 1 only
    assert _plan(ok, [0, 0], xdt=2)[0] == bn.BITNET_ERR_INVALID_ARG          # bf16 or fp32 input
    assert _plan([(256, 512), (512, 384)], [0, 0])[0] == bn.BITNET_ERR_UNSUPPORTED_SHAPE  # K != previous N
    assert _plan([(16384, 128), (128, 8192 + 128)], [0, 1])[0] == bn.BITNET_ERR_UNSUPPORTED_SHAPE  # junction K > 8192
    assert _plan([(256, 16384 + 128)], [0])[0] == bn.BITNET_ERR_UNSUPPORTED_SHAPE   # K > 16384
    assert _plan([(2560, 2560)], [0], cus=16)[0] == bn.BITNET_ERR_UNSUPPORTED_SHAPE  # 40 workgroups > 16 CUs
    assert _plan([(2560, 2560)], [0], cus=40)[0] == bn.BITNET_OK
    L = bn.lib()
    assert L.bitnet_w2a8_chain_persistent(_FAKE, 2, _FAKE, 0, 2, _FAKE, _FAKE, 4096, _NULL) == \
        bn.BITNET_ERR_UNSUPPORTED_SHAPE
    assert L.bitnet_w2a8_chain_persistent(_FAKE, 2, _MIS, 0, 1, _FAKE, _FAKE, 4096, _NULL) == bn.BITNET_ERR_INVALID_ARG
    assert L.bitnet_w2a8_chain_persistent(_FAKE, 2, _FAKE, 3, 1, _FAKE, _FAKE, 4096, _NULL) == bn.BITNET_ERR_INVALID_ARG
    assert L.bitnet_w2a8_chain_persistent_ex(_FAKE, 2, _FAKE, 0, 1, _FAKE, _FAKE, 4096, -1, -1, _NULL) == \
        bn.BITNET_ERR_INVALID_ARG


def _random_valid_chain(rng):
    n = int(rng.integers(2, 9))
    shapes, folds = [], []
    K, fold = 128 * int(rng.integers(1, 129)), 0
    for i in range(n):
        last = i == n - 1
        N = 16 * int(rng.integers(1, 600)) if last else 128 * int(rng.integers(1, 65))
        shapes.append((N, K))
        folds.append(fold)
        if not last:
            fold = int(rng.integers(0, 3)) if (N % 256 == 0 and N // 2 <= 8192) else 0
            K = N // 2 if fold else N
    return shapes, folds


@pytest.mark.parametrize("seed", range(40))
def test_persistent_plan_invariants_on_random_chains(seed):
    """Whatever the chain, the plan covers every row and block, stays within the CU count,
    takes the most row tiles per workgroup that fit, and lays the layer buffers out without
    overlap; inputs past the size limits are refused."""
    rng = np.random.default_rng(np.random.SeedSequence([91, seed]))
    shapes, folds = _random_valid_chain(rng)
    cus = int(rng.choice([40, 104, 256, 256, 304]))
    xdt = int(rng.integers(0, 2))
    st, t, ws = _plan(shapes, folds, 1, xdt, cus)
    too_big = any(K > 16384 or (f and K > 8192) for (N, K), f in zip(shapes, folds))

    def fits(tp, N, K):
        nw, nblk = 16 // tp, K // 128
        per = -(-nblk // nw)
        return per <= 8 and -(-(N // 16) // tp) <= cus

    if too_big or not all(any(fits(tp, N, K) for tp in (4, 2, 1)) for N, K in shapes):
        assert st == bn.BITNET_ERR_UNSUPPORTED_SHAPE
        return
    assert st == bn.BITNET_OK
    offs = t.view(np.int64).reshape(len(shapes), 8)
    end = 256
    for i, ((N, K), f) in enumerate(zip(shapes, folds)):
        Nf, Kf, xm, tp, nw, per, nwg = (int(v) for v in t[i][8:15])
        assert (Nf, Kf) == (N, K)
        assert xm == ((0 if xdt == bn.BITNET_DT_BF16 else 1) if i == 0 else {0: 4, 1: 5, 2: 6}[f])
        assert tp in (1, 2, 4) and nw * tp == 16 and 1 <= per <= 8
        assert per * nw * 128 >= K                      # the waves of a tile cover every block
        assert nwg * tp * 16 >= N and (nwg - 1) * tp * 16 < N and nwg <= cus  # rows covered, none idle
        assert all(not fits(bigger, N, K) for bigger in (4, 2) if bigger > tp)
        if i == 0:
            assert offs[i, 2] == -1
        else:
            assert offs[i, 2] == offs[i - 1, 3]
        if i == len(shapes) - 1:
            assert offs[i, 3] == -1
        else:
            assert offs[i, 3] == end and end % 256 == 0
            end += -(-N * 4 // 256) * 256
    assert ws == end
