"""Python binding of libbitnet_w2a8.so (MI355X / gfx950 W2A8 ternary product).

Argument marshalling only: every step of the path runs in the library's HIP
kernels or, for the offline packer, in its host C++ code.  torch supplies
device memory and streams.  The C ABI and the tile layout are specified in
``include/bitnet_w2a8.h``; the functions below carry the same names.

If the library is not built, every call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitnet_w2a8.so")

BITNET_OK, BITNET_ERR_INVALID_ARG, BITNET_ERR_UNSUPPORTED_SHAPE, BITNET_ERR_HIP = 0, 1, 2, 3
BITNET_DT_BF16, BITNET_DT_F32, BITNET_DT_F32_FOLD2, BITNET_DT_F32_RELU2_GLU = 0, 1, 2, 3
BITNET_JUNCTION_NONE, BITNET_JUNCTION_SUM, BITNET_JUNCTION_RELU2_GLU = 0, 1, 2
_JUNCTIONS = {False: 0, None: 0, "none": 0, True: 1, "sum": 1, "relu2_glu": 2, 0: 0, 1: 1, 2: 2}


def junction_code(j) -> int:
    """Junction of a two-half input: False/None/"none" -> 0, True/"sum" -> 1 (lo + hi),
    "relu2_glu" -> 2 (relu(lo)^2 * hi); the integers 0..2 map to themselves."""
    try:
        return _JUNCTIONS[j]
    except (KeyError, TypeError):
        raise ValueError(f"unknown junction {j!r}") from None
BLOCK_K = 128
TILE_N = 16
GEMV_MAX_M = 16


class BitnetError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {bitnet_status_str(status)} (status {status})")
        self.status = status


_lib = None

_SIGS = {
    "bitnet_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "bitnet_check_shape": ([ctypes.c_int64, ctypes.c_int64], ctypes.c_int),
    "bitnet_gemv_split": ([ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                           ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
    "bitnet_packed_bytes": ([ctypes.c_int64, ctypes.c_int64], ctypes.c_size_t),
    "bitnet_scale_count": ([ctypes.c_int64, ctypes.c_int64], ctypes.c_size_t),
    "bitnet_ternarize_absmean": ([ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_void_p], ctypes.c_int),
    "bitnet_pack_i2s": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                         ctypes.c_void_p], ctypes.c_int),
    "bitnet_repack_i2s": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                           ctypes.c_void_p], ctypes.c_int),
    "bitnet_unpack_i2s": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                           ctypes.c_void_p], ctypes.c_int),
    "bitnet_quant_act": ([ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                          ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "bitnet_quant_act_fold": ([ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p], ctypes.c_int),
    "bitnet_quant_act_relu2_glu": ([ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p], ctypes.c_int),
    "bitnet_w2a8_gemv": ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 3 + [ctypes.c_void_p], ctypes.c_int),
    "bitnet_w2a8_gemm": ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [ctypes.c_void_p], ctypes.c_int),
    "bitnet_scale_count_g": ([ctypes.c_int64, ctypes.c_int64, ctypes.c_int], ctypes.c_size_t),
    "bitnet_probe_stream_read_sink_len": ([ctypes.c_size_t], ctypes.c_size_t),
    "bitnet_probe_stream_read": ([ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                  ctypes.c_void_p], ctypes.c_int),
    "bitnet_ternarize_absmean_g": ([ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p], ctypes.c_int),
    "bitnet_pack_i2s_g": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                           ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "bitnet_repack_i2s_g": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                             ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "bitnet_unpack_i2s_g": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                             ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "bitnet_w2a8_gemv_g": ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [ctypes.c_void_p], ctypes.c_int),
    "bitnet_w2a8_gemm_g": ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_void_p], ctypes.c_int),
    "bitnet_w2a8_gemv_act": ([ctypes.c_void_p] * 3 + [ctypes.c_int] + [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3
                             + [ctypes.c_void_p], ctypes.c_int),
    "bitnet_w2a8_acc_i32": ([ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [ctypes.c_void_p], ctypes.c_int),
    "bitnet_w2a8_gemv_lut": ([ctypes.c_void_p] * 6 + [ctypes.c_int] * 3 + [ctypes.c_void_p], ctypes.c_int),
    "bitnet_w2a8_chain_workspace_bytes": ([ctypes.c_void_p, ctypes.c_int, ctypes.c_int], ctypes.c_size_t),
    "bitnet_w2a8_chain": ([ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                           ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "bitnet_w2a8_chain_static_max_bytes": ([], ctypes.c_size_t),
    "bitnet_w2a8_persist_table_bytes": ([ctypes.c_int], ctypes.c_size_t),
    "bitnet_w2a8_persist_prepare": ([ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "bitnet_w2a8_chain_persistent": ([ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "bitnet_w2a8_chain_persistent_ex": ([ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p], ctypes.c_int),
    "bitnet_w2a8_chain_static": ([ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
}


class ChainLayer(ctypes.Structure):
    """bitnet_chain_layer_t"""
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("N", ctypes.c_int), ("K", ctypes.c_int),
                ("fold_input", ctypes.c_int)]


def lib():
    """The loaded library (ctypes.CDLL).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        # The kernels must run on the HIP runtime that owns the device memory and
        # streams passed in.  torch bundles its own libamdhip64 under the same
        # soname; with torch loaded first the dynamic linker binds this library to
        # that copy, while loading this library first would map the system runtime
        # and torch would then load a second one beside it.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run `python -m bit_gemv_i2_amd.build`)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _ok(status: int, what: str):
    if status != BITNET_OK:
        raise BitnetError(status, what)


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dev_ptr(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _check(t, name: str, dtype, numel: int | None = None, shape: tuple | None = None):
    """Raises ValueError unless tensor t has the given dtype and exactly `numel`
    elements (or exactly `shape`).  Runs on metadata only, before any pointer is
    taken or any launch is made: a buffer whose size disagrees with the library's
    size authorities (bitnet_packed_bytes, bitnet_scale_count[_g], M*K, M*N) is
    never handed to a kernel."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, not {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, not {t.numel()}")


def _check_weights(packed, scales, N: int, K: int, scale_block: int = 128):
    """packed / scales against bitnet_packed_bytes and bitnet_scale_count[_g]."""
    import torch
    nb = bitnet_packed_bytes(N, K)
    ns = bitnet_scale_count(N, K) if scale_block == 128 else bitnet_scale_count_g(N, K, scale_block)
    if nb == 0 or ns == 0:
        raise BitnetError(BITNET_ERR_UNSUPPORTED_SHAPE if nb == 0 else BITNET_ERR_INVALID_ARG,
                          f"weights of shape {N} x {K} (scale_block {scale_block})")
    _check(packed, "packed", torch.uint8, numel=nb)
    if scales is not None:
        _check(scales, "scales", torch.float32, numel=ns)


def _check_acts(q, s_a, K: int):
    """q int8 [M][K] and s_a fp32 [M]; returns M."""
    import torch
    if q.dim() != 2 or q.shape[1] != K:
        raise ValueError(f"q must be [M][{K}], not {tuple(q.shape)}")
    _check(q, "q", torch.int8)
    M = q.shape[0]
    if s_a is not None:
        _check(s_a, "s_a", torch.float32, numel=M)
    return M


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ sizes
def bitnet_status_str(status: int) -> str:
    return lib().bitnet_status_str(int(status)).decode()


def bitnet_check_shape(N: int, K: int) -> int:
    return lib().bitnet_check_shape(N, K)


def bitnet_gemv_split(N: int, K: int, cus: int = 0, wave_slots: int = 0):
    """(waves per 16-row workgroup, 128-weight blocks per wave) of the decode products for an
    N x K matrix on a device with `cus` CUs holding `wave_slots` waves (0, 0: the base split)."""
    w, p = ctypes.c_int(0), ctypes.c_int(0)
    _ok(lib().bitnet_gemv_split(int(N), int(K), int(cus), int(wave_slots), ctypes.byref(w), ctypes.byref(p)),
        "bitnet_gemv_split")
    return w.value, p.value


def bitnet_packed_bytes(N: int, K: int) -> int:
    return lib().bitnet_packed_bytes(N, K)


def bitnet_scale_count(N: int, K: int) -> int:
    return lib().bitnet_scale_count(N, K)


# ------------------------------------------------------------------ offline, host
def bitnet_ternarize_absmean(w: np.ndarray):
    """fp32 [N][K] -> (ternary int8 [N][K], scales fp32 [N][K/128])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    t = np.empty((N, K), np.int8)
    s = np.empty((N, K // BLOCK_K), np.float32)
    _ok(lib().bitnet_ternarize_absmean(_np_ptr(w), N, K, _np_ptr(t), _np_ptr(s)), "bitnet_ternarize_absmean")
    return t, s


def bitnet_pack_i2s(ternary: np.ndarray, scales: np.ndarray):
    """ternary int8 [N][K], scales fp32 [N][K/128] -> (packed uint8 [N*K/4], tiled scales fp32 [N*K/128])."""
    ternary = np.ascontiguousarray(ternary, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    N, K = ternary.shape
    if scales.shape != (N, K // BLOCK_K):
        raise ValueError("scales must be [N][K/128]")
    nb = bitnet_packed_bytes(N, K)
    if nb == 0:
        raise BitnetError(BITNET_ERR_UNSUPPORTED_SHAPE, "bitnet_pack_i2s")
    packed = np.empty(nb, np.uint8)
    st = np.empty(bitnet_scale_count(N, K), np.float32)
    _ok(lib().bitnet_pack_i2s(_np_ptr(ternary), _np_ptr(scales), N, K, _np_ptr(packed), _np_ptr(st)),
        "bitnet_pack_i2s")
    return packed, st


def bitnet_repack_i2s(i2s: np.ndarray, scales: np.ndarray, K: int):
    """canonical i2_s bytes uint8 [N][K/4] + scales [N][K/128] -> (packed, tiled scales)."""
    i2s = np.ascontiguousarray(i2s, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    N = i2s.shape[0]
    if i2s.shape != (N, K // 4) or scales.shape != (N, K // BLOCK_K):
        raise ValueError("bad i2s / scales shape")
    nb = bitnet_packed_bytes(N, K)
    if nb == 0:
        raise BitnetError(BITNET_ERR_UNSUPPORTED_SHAPE, "bitnet_repack_i2s")
    packed = np.empty(nb, np.uint8)
    st = np.empty(bitnet_scale_count(N, K), np.float32)
    _ok(lib().bitnet_repack_i2s(_np_ptr(i2s), _np_ptr(scales), N, K, _np_ptr(packed), _np_ptr(st)),
        "bitnet_repack_i2s")
    return packed, st


def bitnet_unpack_i2s(packed: np.ndarray, scales_tiled: np.ndarray | None, N: int, K: int):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    t = np.empty((N, K), np.int8)
    s = None
    sp = None
    if scales_tiled is not None:
        scales_tiled = np.ascontiguousarray(scales_tiled, dtype=np.float32)
        s = np.empty((N, K // BLOCK_K), np.float32)
        sp = _np_ptr(scales_tiled)
    _ok(lib().bitnet_unpack_i2s(_np_ptr(packed), sp, N, K, _np_ptr(t), None if s is None else _np_ptr(s)),
        "bitnet_unpack_i2s")
    return t, s


# ------------------------------------------------------------------ scale granularity
# scale_block: 128 (x86 i2_s blocks, the default everywhere else), 64 (ARM
# blocks) or 0 (one scale for the whole matrix).
def scale_shape(N: int, K: int, scale_block: int):
    return (1,) if scale_block == 0 else (N, K // scale_block)


def bitnet_scale_count_g(N: int, K: int, scale_block: int) -> int:
    return lib().bitnet_scale_count_g(N, K, scale_block)


def bitnet_ternarize_absmean_g(w: np.ndarray, scale_block: int):
    """fp32 [N][K] -> (ternary int8 [N][K], scales fp32 scale_shape(N, K, scale_block))."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    t = np.empty((N, K), np.int8)
    s = np.empty(scale_shape(N, K, scale_block), np.float32)
    _ok(lib().bitnet_ternarize_absmean_g(_np_ptr(w), N, K, scale_block, _np_ptr(t), _np_ptr(s)),
        "bitnet_ternarize_absmean_g")
    return t, s


def _pack_g(name, src, scales, N, K, scale_block):
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    if scales.shape != scale_shape(N, K, scale_block):
        raise ValueError("scales must have shape %s" % (scale_shape(N, K, scale_block),))
    nb, ns = bitnet_packed_bytes(N, K), bitnet_scale_count_g(N, K, scale_block)
    if nb == 0 or ns == 0:
        raise BitnetError(BITNET_ERR_UNSUPPORTED_SHAPE, name)
    packed = np.empty(nb, np.uint8)
    st = np.empty(ns, np.float32)
    _ok(getattr(lib(), name)(_np_ptr(src), _np_ptr(scales), N, K, scale_block, _np_ptr(packed), _np_ptr(st)), name)
    return packed, st


def bitnet_pack_i2s_g(ternary: np.ndarray, scales: np.ndarray, scale_block: int):
    """As bitnet_pack_i2s, scales of shape scale_shape(N, K, scale_block)."""
    ternary = np.ascontiguousarray(ternary, dtype=np.int8)
    N, K = ternary.shape
    return _pack_g("bitnet_pack_i2s_g", ternary, scales, N, K, scale_block)


def bitnet_repack_i2s_g(i2s: np.ndarray, scales: np.ndarray, K: int, scale_block: int):
    """Canonical bytes of the given format uint8 [N][K/4] + scales -> (packed, tiled scales)."""
    i2s = np.ascontiguousarray(i2s, dtype=np.uint8)
    N = i2s.shape[0]
    if i2s.shape != (N, K // 4):
        raise ValueError("bad i2s shape")
    return _pack_g("bitnet_repack_i2s_g", i2s, scales, N, K, scale_block)


def bitnet_unpack_i2s_g(packed: np.ndarray, scales_tiled, N: int, K: int, scale_block: int):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    t = np.empty((N, K), np.int8)
    s = sp = None
    if scales_tiled is not None:
        scales_tiled = np.ascontiguousarray(scales_tiled, dtype=np.float32)
        s = np.empty(scale_shape(N, K, scale_block), np.float32)
        sp = _np_ptr(scales_tiled)
    _ok(lib().bitnet_unpack_i2s_g(_np_ptr(packed), sp, N, K, scale_block, _np_ptr(t),
                                  None if s is None else _np_ptr(s)), "bitnet_unpack_i2s_g")
    return t, s


# ------------------------------------------------------------------ device, async
def bitnet_quant_act(x, q=None, s_a=None, stream=None):
    """x: device [M][K] bf16 or fp32 -> (q int8 [M][K], s_a fp32 [M])."""
    import torch
    M, K = x.shape
    xdt = {torch.bfloat16: BITNET_DT_BF16, torch.float32: BITNET_DT_F32}.get(x.dtype)
    if xdt is None:
        raise ValueError("x must be bf16 or fp32")
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s_a is None:
        s_a = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(q, "q", torch.int8, numel=M * K)
    _check(s_a, "s_a", torch.float32, numel=M)
    _ok(lib().bitnet_quant_act(_dev_ptr(x, "x"), xdt, M, K, _dev_ptr(q, "q"), _dev_ptr(s_a, "s_a"),
                               _stream(stream)), "bitnet_quant_act")
    return q, s_a


def _quant_two_half(name, y, q, s_a, stream):
    import torch
    M, H2 = y.shape
    H = H2 // 2
    if y.dtype != torch.float32 or H2 % 2:
        raise ValueError("y must be fp32 [M][2H]")
    if q is None:
        q = torch.empty((M, H), dtype=torch.int8, device=y.device)
    if s_a is None:
        s_a = torch.empty((M,), dtype=torch.float32, device=y.device)
    _check(q, "q", torch.int8, numel=M * H)
    _check(s_a, "s_a", torch.float32, numel=M)
    _ok(getattr(lib(), name)(_dev_ptr(y, "y"), M, H, _dev_ptr(q, "q"), _dev_ptr(s_a, "s_a"), _stream(stream)), name)
    return q, s_a


def bitnet_quant_act_fold(y, q=None, s_a=None, stream=None):
    """y: device fp32 [M][2H] -> h = y[:, :H] + y[:, H:] quantised: (q int8 [M][H], s_a fp32 [M])."""
    return _quant_two_half("bitnet_quant_act_fold", y, q, s_a, stream)


def bitnet_quant_act_relu2_glu(y, q=None, s_a=None, stream=None):
    """y: device fp32 [M][2H] (gate | up) -> h = relu(gate)^2 * up quantised: (q int8 [M][H], s_a fp32 [M])."""
    return _quant_two_half("bitnet_quant_act_relu2_glu", y, q, s_a, stream)


def bitnet_w2a8_gemv(packed, scales, q, s_a, N: int, K: int, y=None, stream=None):
    """Decode product (M <= 16): y fp32 [M][N]."""
    import torch
    _check_weights(packed, scales, N, K)
    M = _check_acts(q, s_a, K)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=q.device)
    _check(y, "y", torch.float32, numel=M * N)
    _ok(lib().bitnet_w2a8_gemv(_dev_ptr(packed, "packed"), _dev_ptr(scales, "scales"), _dev_ptr(q, "q"),
                               _dev_ptr(s_a, "s_a"), _dev_ptr(y, "y"), M, N, K, _stream(stream)),
        "bitnet_w2a8_gemv")
    return y


def bitnet_w2a8_gemv_act(packed, scales, x, N: int, K: int, fold: bool = False, y=None, q_out=None,
                         s_a_out=None, stream=None):
    """Decode step in one launch: quantise x (bf16/fp32 [M][K], or fp32 [M][2K]
    brought to width K by a junction: fold=True or "sum" for lo + hi,
    "relu2_glu" for relu(lo)^2 * hi) and multiply.  Optional q_out / s_a_out
    receive the int8 activations and dequant factors.  Returns y fp32 [M][N]."""
    import torch
    M = x.shape[0]
    jc = junction_code(fold)
    if jc:
        if x.dtype != torch.float32 or x.shape[1] != 2 * K:
            raise ValueError("a junction needs fp32 x of shape [M][2K]")
        xdt = BITNET_DT_F32_FOLD2 if jc == BITNET_JUNCTION_SUM else BITNET_DT_F32_RELU2_GLU
    else:
        xdt = {torch.bfloat16: BITNET_DT_BF16, torch.float32: BITNET_DT_F32}.get(x.dtype)
        if xdt is None or x.shape[1] != K:
            raise ValueError("x must be bf16 or fp32 [M][K]")
    _check_weights(packed, scales, N, K)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check(y, "y", torch.float32, numel=M * N)
    if q_out is not None:
        _check(q_out, "q_out", torch.int8, numel=M * K)
    if s_a_out is not None:
        _check(s_a_out, "s_a_out", torch.float32, numel=M)
    qp = None if q_out is None else _dev_ptr(q_out, "q_out")
    sp = None if s_a_out is None else _dev_ptr(s_a_out, "s_a_out")
    _ok(lib().bitnet_w2a8_gemv_act(_dev_ptr(packed, "packed"), _dev_ptr(scales, "scales"), _dev_ptr(x, "x"), xdt,
                                   _dev_ptr(y, "y"), qp, sp, M, N, K, _stream(stream)), "bitnet_w2a8_gemv_act")
    return y


def bitnet_w2a8_gemm(packed, scales, q, s_a, N: int, K: int, out_dtype=None, y=None, stream=None):
    """Prefill product (any M): y [M][N] in bf16 (default) or fp32."""
    import torch
    _check_weights(packed, scales, N, K)
    M = _check_acts(q, s_a, K)
    if out_dtype is None:
        out_dtype = torch.bfloat16 if y is None else y.dtype
    ydt = {torch.bfloat16: BITNET_DT_BF16, torch.float32: BITNET_DT_F32}.get(out_dtype)
    if ydt is None:
        raise ValueError("out_dtype must be bf16 or fp32")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=q.device)
    _check(y, "y", out_dtype, numel=M * N)
    _ok(lib().bitnet_w2a8_gemm(_dev_ptr(packed, "packed"), _dev_ptr(scales, "scales"), _dev_ptr(q, "q"),
                               _dev_ptr(s_a, "s_a"), _dev_ptr(y, "y"), ydt, M, N, K, _stream(stream)),
        "bitnet_w2a8_gemm")
    return y


def bitnet_w2a8_gemv_g(packed, scales, q, s_a, N: int, K: int, scale_block: int, y=None, stream=None):
    """Decode product at scale granularity scale_block (tiled scales of bitnet_pack_i2s_g)."""
    import torch
    _check_weights(packed, scales, N, K, scale_block)
    M = _check_acts(q, s_a, K)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=q.device)
    _check(y, "y", torch.float32, numel=M * N)
    _ok(lib().bitnet_w2a8_gemv_g(_dev_ptr(packed, "packed"), _dev_ptr(scales, "scales"), _dev_ptr(q, "q"),
                                 _dev_ptr(s_a, "s_a"), _dev_ptr(y, "y"), M, N, K, scale_block, _stream(stream)),
        "bitnet_w2a8_gemv_g")
    return y


def bitnet_w2a8_gemm_g(packed, scales, q, s_a, N: int, K: int, scale_block: int, out_dtype=None, y=None,
                       stream=None):
    """Prefill product at scale granularity scale_block."""
    import torch
    _check_weights(packed, scales, N, K, scale_block)
    M = _check_acts(q, s_a, K)
    if out_dtype is None:
        out_dtype = torch.bfloat16 if y is None else y.dtype
    ydt = {torch.bfloat16: BITNET_DT_BF16, torch.float32: BITNET_DT_F32}.get(out_dtype)
    if ydt is None:
        raise ValueError("out_dtype must be bf16 or fp32")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=q.device)
    _check(y, "y", out_dtype, numel=M * N)
    _ok(lib().bitnet_w2a8_gemm_g(_dev_ptr(packed, "packed"), _dev_ptr(scales, "scales"), _dev_ptr(q, "q"),
                                 _dev_ptr(s_a, "s_a"), _dev_ptr(y, "y"), ydt, M, N, K, scale_block,
                                 _stream(stream)), "bitnet_w2a8_gemm_g")
    return y


def bitnet_w2a8_acc_i32(packed, q, N: int, K: int, acc=None, stream=None):
    """Exact int32 product acc [M][N] through the decode (M <= 16) or prefill kernel."""
    import torch
    _check_weights(packed, None, N, K)
    M = _check_acts(q, None, K)
    if acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=q.device)
    _check(acc, "acc", torch.int32, numel=M * N)
    _ok(lib().bitnet_w2a8_acc_i32(_dev_ptr(packed, "packed"), _dev_ptr(q, "q"), _dev_ptr(acc, "acc"), M, N, K,
                                  _stream(stream)), "bitnet_w2a8_acc_i32")
    return acc


def bitnet_w2a8_gemv_lut(packed, scales, q, s_a, N: int, K: int, tiles_per_group: int = 0, y=None, acc=None,
                         with_acc: bool = False, stream=None):
    """Table-lookup decode product for one token: y fp32 [1][N] (and, with
    with_acc or a given acc, the exact int32 sums [1][N]).  Returns y, or (y, acc)."""
    import torch
    if q.dim() != 2 or q.shape[0] != 1:
        raise ValueError("q must be int8 [1][K]")
    _check_weights(packed, scales, N, K)
    _check_acts(q, s_a, K)
    if y is None:
        y = torch.empty((1, N), dtype=torch.float32, device=q.device)
    if acc is None and with_acc:
        acc = torch.empty((1, N), dtype=torch.int32, device=q.device)
    _check(y, "y", torch.float32, numel=N)
    if acc is not None:
        _check(acc, "acc", torch.int32, numel=N)
    accp = _dev_ptr(acc, "acc") if acc is not None else None
    _ok(lib().bitnet_w2a8_gemv_lut(_dev_ptr(packed, "packed"), _dev_ptr(scales, "scales"), _dev_ptr(q, "q"),
                                   _dev_ptr(s_a, "s_a"), _dev_ptr(y, "y"), accp, N, K, tiles_per_group,
                                   _stream(stream)), "bitnet_w2a8_gemv_lut")
    return (y, acc) if acc is not None else y


# ------------------------------------------------------------------ convenience
@dataclass
class PackedWeight:
    """A ternary weight matrix resident in device memory in the tile layout."""
    packed: object   # torch uint8 [N*K/4] on device
    scales: object   # torch fp32 [N*K/128] on device (tiled order)
    N: int
    K: int

    @classmethod
    def from_ternary(cls, ternary: np.ndarray, scales: np.ndarray, device="cuda"):
        import torch
        p, s = bitnet_pack_i2s(ternary, scales)
        N, K = ternary.shape
        return cls(torch.from_numpy(p).to(device), torch.from_numpy(s).to(device), N, K)

    def gemv(self, q, s_a, y=None, stream=None):
        return bitnet_w2a8_gemv(self.packed, self.scales, q, s_a, self.N, self.K, y=y, stream=stream)

    def gemv_act(self, x, fold=False, y=None, q_out=None, s_a_out=None, stream=None):
        return bitnet_w2a8_gemv_act(self.packed, self.scales, x, self.N, self.K, fold=fold, y=y, q_out=q_out,
                                    s_a_out=s_a_out, stream=stream)

    def gemm(self, q, s_a, out_dtype=None, y=None, stream=None):
        return bitnet_w2a8_gemm(self.packed, self.scales, q, s_a, self.N, self.K, out_dtype=out_dtype, y=y,
                                stream=stream)


# ------------------------------------------------------------------ chained decode
class Chain:
    """A stack of W2A8 layers run by bitnet_w2a8_chain.  `weights` are
    PackedWeight objects; `folds[i]` is the junction in front of layer i
    (False: none; True or "sum": previous output folded h = lo + hi;
    "relu2_glu": h = relu(lo)^2 * hi)."""

    def __init__(self, weights, folds=None):
        self.weights = list(weights)
        self.folds = [0] * len(self.weights) if folds is None else [junction_code(f) for f in folds]
        n = len(self.weights)
        self._arr = (ChainLayer * n)()
        for i, (w, f) in enumerate(zip(self.weights, self.folds)):
            self._arr[i] = ChainLayer(w.packed.data_ptr(), w.scales.data_ptr(), w.N, w.K, int(f))
        self._ws = {}

    def workspace_bytes(self, M: int) -> int:
        return lib().bitnet_w2a8_chain_workspace_bytes(ctypes.cast(self._arr, ctypes.c_void_p), len(self.weights), M)

    def workspace(self, M: int, device="cuda"):
        import torch
        if M not in self._ws:
            nb = self.workspace_bytes(M)
            if nb == 0:
                raise BitnetError(BITNET_ERR_UNSUPPORTED_SHAPE, "bitnet_w2a8_chain_workspace_bytes")
            self._ws[M] = torch.empty(nb, dtype=torch.uint8, device=device)
        return self._ws[M]

    def __call__(self, x, y=None, stream=None):
        import torch
        M = x.shape[0]
        xdt = {torch.bfloat16: BITNET_DT_BF16, torch.float32: BITNET_DT_F32}.get(x.dtype)
        if xdt is None:
            raise ValueError("x must be bf16 or fp32")
        if x.dim() != 2 or x.shape[1] != self.weights[0].K:
            raise ValueError(f"x must be [M][{self.weights[0].K}], not {tuple(x.shape)}")
        if y is None:
            y = torch.empty((M, self.weights[-1].N), dtype=torch.float32, device=x.device)
        _check(y, "y", torch.float32, numel=M * self.weights[-1].N)
        ws = self.workspace(M, x.device)
        _ok(lib().bitnet_w2a8_chain(ctypes.cast(self._arr, ctypes.c_void_p), len(self.weights), _dev_ptr(x, "x"), xdt,
                                    M, _dev_ptr(y, "y"), _dev_ptr(ws, "workspace"), ws.numel(), _stream(stream)),
            "bitnet_w2a8_chain")
        return y


    def plan_persistent(self, M: int = 1, xdt: int = BITNET_DT_BF16, cus: int = 0, device="cuda"):
        key = ("persistent", M, xdt, cus)
        if key not in self._ws:
            self._ws[key] = PersistentPlan(self, M, xdt, cus, device)
        return self._ws[key]

    def persistent(self, x, y=None, stream=None, workspace=None, spin_limit: int = 0, withhold: int = -1):
        """The same decode pass as one persistent launch (bitnet_w2a8_chain_persistent, batch 1).
        Returns y; the workspace (which the binding allocates unless one is given) then
        holds the status word (int32 at offset 0: 0; the layer index + 1 of a wait that
        gave up; minus (layer index + 1) of a table entry that does not fit the workspace)
        and every intermediate layer's output.  spin_limit / withhold are the
        test-only knobs of bitnet_w2a8_chain_persistent_ex."""
        import torch
        M = x.shape[0]
        xdt = {torch.bfloat16: BITNET_DT_BF16, torch.float32: BITNET_DT_F32}.get(x.dtype)
        if xdt is None:
            raise ValueError("x must be bf16 or fp32")
        if x.dim() != 2 or x.shape[1] != self.weights[0].K:
            raise ValueError(f"x must be [M][{self.weights[0].K}], not {tuple(x.shape)}")
        plan = self.plan_persistent(M, xdt, device=x.device)
        if y is None:
            y = torch.empty((M, self.weights[-1].N), dtype=torch.float32, device=x.device)
        _check(y, "y", torch.float32, numel=M * self.weights[-1].N)
        if workspace is None:
            wkey = ("persistent_ws", M, xdt)
            if wkey not in self._ws:
                self._ws[wkey] = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=x.device)
            workspace = self._ws[wkey]
        _check(workspace, "workspace", torch.uint8)
        if workspace.numel() < plan.workspace_bytes:
            raise ValueError(f"workspace must hold at least {plan.workspace_bytes} bytes")
        _ok(lib().bitnet_w2a8_chain_persistent_ex(_dev_ptr(plan.table, "table"), plan.n, _dev_ptr(x, "x"), xdt, M,
                                                  _dev_ptr(y, "y"), _dev_ptr(workspace, "workspace"),
                                                  workspace.numel(), int(spin_limit), int(withhold), _stream(stream)),
            "bitnet_w2a8_chain_persistent")
        return y

    def persistent_layer_outputs(self, M: int = 1, xdt: int = BITNET_DT_BF16, workspace=None):
        """Host views (fp32 [M][N]) of every intermediate layer's output as the last
        persistent call left them in its workspace (the caller's, if one was passed to that
        call, else the binding's), and the status word."""
        plan = self.plan_persistent(M, xdt)
        if workspace is None:
            key = ("persistent_ws", M, xdt)
            if key not in self._ws:
                raise ValueError("no persistent call with the binding's workspace has been made for this batch and type")
            workspace = self._ws[key]
        import torch
        _check(workspace, "workspace", torch.uint8)
        if workspace.numel() < plan.workspace_bytes:
            raise ValueError(f"workspace must hold at least {plan.workspace_bytes} bytes")
        ws = workspace.cpu().numpy()
        table = plan.host_table.view(np.int64).reshape(plan.n, 8)  # out_off is the 4th 8-byte field
        outs = []
        for i in range(plan.n - 1):
            off = int(table[i, 3])
            N = self.weights[i].N
            outs.append(ws[off:off + 4 * M * N].view(np.float32).reshape(M, N).copy())
        return outs, int(ws[:4].view(np.int32)[0])

    def call_static(self, x, y=None, stream=None):
        """The same pass through bitnet_w2a8_chain_static: no workspace is allocated (the
        library's per-GPU array serves), for callers that cannot allocate."""
        import torch
        M = x.shape[0]
        xdt = {torch.bfloat16: BITNET_DT_BF16, torch.float32: BITNET_DT_F32}.get(x.dtype)
        if xdt is None:
            raise ValueError("x must be bf16 or fp32")
        if x.dim() != 2 or x.shape[1] != self.weights[0].K:
            raise ValueError(f"x must be [M][{self.weights[0].K}], not {tuple(x.shape)}")
        if y is None:
            y = torch.empty((M, self.weights[-1].N), dtype=torch.float32, device=x.device)
        _check(y, "y", torch.float32, numel=M * self.weights[-1].N)
        _ok(lib().bitnet_w2a8_chain_static(ctypes.cast(self._arr, ctypes.c_void_p), len(self.weights),
                                           _dev_ptr(x, "x"), xdt, M, _dev_ptr(y, "y"), _stream(stream)),
            "bitnet_w2a8_chain_static")
        return y


class PersistentPlan:
    """The layer table and workspace size of the one-launch (persistent) form of a chain,
    from bitnet_w2a8_persist_prepare (host), with the table copied to the device once:
    the weights' addresses are fixed, so a plan serves every later call."""

    def __init__(self, chain: "Chain", M: int, xdt: int, cus: int = 0, device="cuda"):
        import torch
        n = len(chain.weights)
        nb = lib().bitnet_w2a8_persist_table_bytes(n)
        host = np.zeros(nb, np.uint8)
        ws = ctypes.c_size_t(0)
        _ok(lib().bitnet_w2a8_persist_prepare(ctypes.cast(chain._arr, ctypes.c_void_p), n, M, xdt, cus,
                                              _np_ptr(host), nb, ctypes.byref(ws)), "bitnet_w2a8_persist_prepare")
        self.host_table = host
        self.table = torch.from_numpy(host).to(device)
        self.workspace_bytes = ws.value
        self.n = n


def bitnet_w2a8_chain_static_max_bytes() -> int:
    return lib().bitnet_w2a8_chain_static_max_bytes()


# ------------------------------------------------------------------ measurement helper
def bitnet_probe_stream_read(src, sink=None, mode=0, stream=None):
    """One pass of 16-byte non-temporal loads over the device tensor `src` (not part of
    the product path; the benchmark's attainable-bandwidth reference).  mode 0:
    returns the uint32 sink whose sum (mod 2^32) is the sum of src's 32-bit
    words; mode 1: no output (the read-only floor), the sink is left as it was."""
    import torch
    nbytes = src.numel() * src.element_size()
    nsink = lib().bitnet_probe_stream_read_sink_len(nbytes)
    if sink is None:
        sink = torch.empty((nsink,), dtype=torch.int32, device=src.device)
    _check(sink, "sink", torch.int32)
    if sink.numel() < nsink:
        raise ValueError(f"sink must hold at least {nsink} entries, not {sink.numel()}")
    _ok(lib().bitnet_probe_stream_read(_dev_ptr(src, "src"), nbytes, _dev_ptr(sink, "sink"), sink.numel(), int(mode),
                                       _stream(stream)), "bitnet_probe_stream_read")
    return sink
