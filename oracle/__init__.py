"""CPU oracle for the W2A8 ternary product -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (``bit_gemv_i2_amd``) never imports
it and shares no code with it.  Every function here is a thin numpy wrapper
over a plain C routine in ``oracle.c``; the arithmetic and its citations of
the pages live there:

* [P2] "5x performance leap: BitNet vs llama.cpp" -- W2A8 = 2-bit weights x
  8-bit activations ("Architecture foundations", item 2).
* [P3] "BitNet + WebAssembly" -- ternary weights from absmean quantisation
  ("Why WASM"), the i2_s code map, 4 codes per byte, 128-weight blocks with
  one float scale ("What i2_s actually is").

Parity is pinned, not self-referential: see ``tests/test_oracle_pins.py``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build(force=True)
        lib = ctypes.CDLL(path)
        i64 = ctypes.c_int64
        p = ctypes.c_void_p
        sig = {
            "oracle_ternarize_absmean": [p, i64, i64, p, p],
            "oracle_pack_i2s": [p, i64, i64, p],
            "oracle_unpack_i2s": [p, i64, i64, p],
            "oracle_quant_act_f32": [p, i64, i64, p, p],
            "oracle_quant_act_bf16": [p, i64, i64, p, p, p],
            "oracle_w2a8": [p, p, p, p, i64, i64, i64, p, p, p, p],
            "oracle_acc_dense": [p, p, i64, i64, i64, p],
            "oracle_f32_to_bf16": [p, i64, p],
            "oracle_fold_quant": [p, i64, i64, p, p, p],
            "oracle_glu_quant": [p, i64, i64, p, p, p],
            "oracle_ternarize_absmean_g": [p, i64, i64, ctypes.c_int, p, p],
            "oracle_pack_i2s_g": [p, i64, i64, ctypes.c_int, p],
            "oracle_unpack_i2s_g": [p, i64, i64, ctypes.c_int, p],
            "oracle_w2a8_g": [p, p, p, p, i64, i64, i64, ctypes.c_int, p, p, p, p],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its input (rc={rc})")


def ternarize_absmean(W):
    """fp32 [N][K] -> (T int8 [N][K], S fp32 [N][K/128])."""
    W = _c(W, np.float32)
    N, K = W.shape
    T = np.empty((N, K), np.int8)
    S = np.empty((N, K // 128), np.float32)
    _check(_load().oracle_ternarize_absmean(_ptr(W), N, K, _ptr(T), _ptr(S)), "ternarize")
    return T, S


def pack_i2s(T):
    """Ternary int8 [N][K] -> canonical i2_s bytes uint8 [N][K/4]."""
    T = _c(T, np.int8)
    N, K = T.shape
    P = np.empty((N, K // 4), np.uint8)
    _check(_load().oracle_pack_i2s(_ptr(T), N, K, _ptr(P)), "pack_i2s")
    return P


def unpack_i2s(P, K):
    P = _c(P, np.uint8)
    N = P.shape[0]
    T = np.empty((N, K), np.int8)
    _check(_load().oracle_unpack_i2s(_ptr(P), N, K, _ptr(T)), "unpack_i2s")
    return T


def quant_act_f32(x):
    """fp32 [M][K] -> (q int8 [M][K], s_a fp32 [M])."""
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    _check(_load().oracle_quant_act_f32(_ptr(x), M, K, _ptr(q), _ptr(s)), "quant_act_f32")
    return q, s


def quant_act_bf16(xbits):
    """bf16 bit patterns uint16 [M][K] -> (q int8 [M][K], s_a fp32 [M])."""
    xbits = _c(xbits, np.uint16)
    M, K = xbits.shape
    q = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    scratch = np.empty((M, K), np.float32)
    _check(_load().oracle_quant_act_bf16(_ptr(xbits), M, K, _ptr(q), _ptr(s), _ptr(scratch)),
           "quant_act_bf16")
    return q, s


def w2a8(P, S, Q, s_a, N, K):
    """Canonical i2_s product.  Returns dict(acc int32 [M][N], y64 fp64,
    y fp32, mag fp64)."""
    P = _c(P, np.uint8)
    S = _c(S, np.float32)
    Q = _c(Q, np.int8)
    s_a = _c(s_a, np.float32)
    M = Q.shape[0]
    assert P.shape == (N, K // 4) and S.shape == (N, K // 128) and Q.shape == (M, K)
    acc = np.empty((M, N), np.int32)
    y64 = np.empty((M, N), np.float64)
    y = np.empty((M, N), np.float32)
    mag = np.empty((M, N), np.float64)
    _check(_load().oracle_w2a8(_ptr(P), _ptr(S), _ptr(Q), _ptr(s_a), M, N, K,
                               _ptr(acc), _ptr(y64), _ptr(y), _ptr(mag)), "w2a8")
    return {"acc": acc, "y64": y64, "y": y, "mag": mag}


def acc_dense(T, Q):
    T = _c(T, np.int8)
    Q = _c(Q, np.int8)
    N, K = T.shape
    M = Q.shape[0]
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_acc_dense(_ptr(T), _ptr(Q), M, N, K, _ptr(acc)), "acc_dense")
    return acc


def f32_to_bf16(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _check(_load().oracle_f32_to_bf16(_ptr(x), x.size, _ptr(out)), "f32_to_bf16")
    return out


def fold_quant(y):
    """y fp32 [M][2H] -> h = y[:, :H] + y[:, H:] -> (q int8 [M][H], s_a fp32 [M])."""
    y = _c(y, np.float32)
    M, H2 = y.shape
    H = H2 // 2
    q = np.empty((M, H), np.int8)
    s = np.empty((M,), np.float32)
    scratch = np.empty((M, H), np.float32)
    _check(_load().oracle_fold_quant(_ptr(y), M, H, _ptr(q), _ptr(s), _ptr(scratch)), "fold_quant")
    return q, s


def glu_quant(y):
    """y fp32 [M][2H] (gate | up) -> h = relu(gate)^2 * up -> (q int8 [M][H], s_a fp32 [M])."""
    y = _c(y, np.float32)
    M, H2 = y.shape
    H = H2 // 2
    q = np.empty((M, H), np.int8)
    s = np.empty((M,), np.float32)
    scratch = np.empty((M, H), np.float32)
    _check(_load().oracle_glu_quant(_ptr(y), M, H, _ptr(q), _ptr(s), _ptr(scratch)), "glu_quant")
    return q, s


# ---------------------------------------------------------------- scale granularity G
# G = 128 (x86 block), 64 (ARM block) or 0 (one scale for the whole matrix).
def scale_shape(N, K, G):
    return (1,) if G == 0 else (N, K // G)


def ternarize_absmean_g(W, G):
    """fp32 [N][K] -> (T int8 [N][K], S fp32 scale_shape(N, K, G))."""
    W = _c(W, np.float32)
    N, K = W.shape
    T = np.empty((N, K), np.int8)
    S = np.empty(scale_shape(N, K, G), np.float32)
    _check(_load().oracle_ternarize_absmean_g(_ptr(W), N, K, G, _ptr(T), _ptr(S)), "ternarize_g")
    return T, S


def pack_i2s_g(T, G):
    """Ternary int8 [N][K] -> canonical bytes uint8 [N][K/4] for granularity G."""
    T = _c(T, np.int8)
    N, K = T.shape
    P = np.empty((N, K // 4), np.uint8)
    _check(_load().oracle_pack_i2s_g(_ptr(T), N, K, G, _ptr(P)), "pack_i2s_g")
    return P


def unpack_i2s_g(P, K, G):
    P = _c(P, np.uint8)
    N = P.shape[0]
    T = np.empty((N, K), np.int8)
    _check(_load().oracle_unpack_i2s_g(_ptr(P), N, K, G, _ptr(T)), "unpack_i2s_g")
    return T


def w2a8_g(P, S, Q, s_a, N, K, G):
    """Product with scale granularity G over canonical bytes for G; as w2a8."""
    P = _c(P, np.uint8)
    S = _c(S, np.float32)
    Q = _c(Q, np.int8)
    s_a = _c(s_a, np.float32)
    M = Q.shape[0]
    assert P.shape == (N, K // 4) and S.shape == scale_shape(N, K, G) and Q.shape == (M, K)
    acc = np.empty((M, N), np.int32)
    y64 = np.empty((M, N), np.float64)
    y = np.empty((M, N), np.float32)
    mag = np.empty((M, N), np.float64)
    _check(_load().oracle_w2a8_g(_ptr(P), _ptr(S), _ptr(Q), _ptr(s_a), M, N, K, G,
                                 _ptr(acc), _ptr(y64), _ptr(y), _ptr(mag)), "w2a8_g")
    return {"acc": acc, "y64": y64, "y": y, "mag": mag}
