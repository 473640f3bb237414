"""Device outputs stay inside their buffers.

[P4] "Matrix memory bounds and stride safety" describes a packed 2-bit kernel that
wrote past its tensor when the reader and the kernel disagreed on a stride.  Here
every kernel family writes its outputs into a view of a larger buffer whose bytes
before and after the view hold a canary pattern, at ragged token counts and row
counts (16-row tiles in odd numbers, token tiles cut short, 4- and 16-byte vector
stores at the tails); the canaries must be intact afterwards, and the values must
equal those of the same call into ordinary tensors."""
import ctypes

import numpy as np
import pytest

import bit_gemv_i2_amd as bn
import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
PAD = 4096          # canary bytes on each side (keeps the view 16-byte aligned)
CANARY = 0xA5


class Guarded:
    """A device tensor of `shape` / `dtype` placed between two canary bands."""

    def __init__(self, shape, dtype):
        self.nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((PAD + self.nbytes + PAD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[PAD:PAD + self.nbytes].view(dtype).view(*shape)

    def check(self, what):
        torch.cuda.synchronize()
        h = self.buf.cpu().numpy()
        before = np.count_nonzero(h[:PAD] != CANARY)
        after = np.count_nonzero(h[PAD + self.nbytes:] != CANARY)
        assert before == 0 and after == 0, f"{what}: {before} bytes before and {after} after the output were written"


def same(a, b, what):
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().view(torch.uint8).numpy(), b.cpu().view(torch.uint8).numpy()), what


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def weights(M, N, K, seed=0, G=128):
    c = wl.small_case(seed + M + N + K, M, N, K)
    if G == 128:
        p, s = bn.bitnet_pack_i2s(c.T, c.S)
    else:
        S = wl.rng_for(5, N, K, G).uniform(0.5, 2, size=(1,) if G == 0 else (N, K // G)).astype(np.float32)
        p, s = bn.bitnet_pack_i2s_g(c.T, S, G)
    x = dev(c.x_bits.view(np.int16)).view(torch.bfloat16)
    q, sa = bn.bitnet_quant_act(x)
    return dev(p), dev(s), x, q, sa


@pytest.mark.parametrize("M,K", [(3, 2576), (17, 400), (1, 16)])
@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float32])
def test_quant_outputs_stay_in_bounds(gpu, M, K, xdt):
    x = dev(wl.rng_for(1, M, K).standard_normal((M, K)).astype(np.float32)).to(xdt)
    gq, gs = Guarded((M, K), torch.int8), Guarded((M,), torch.float32)
    bn.bitnet_quant_act(x, gq.t, gs.t)
    gq.check("quant q")
    gs.check("quant s_a")
    q, s = bn.bitnet_quant_act(x)
    same(gq.t, q, "quant q")
    same(gs.t, s, "quant s_a")


@pytest.mark.parametrize("fn", [bn.bitnet_quant_act_fold, bn.bitnet_quant_act_relu2_glu])
@pytest.mark.parametrize("M,H", [(3, 2576), (5, 48)])
def test_junction_quant_outputs_stay_in_bounds(gpu, fn, M, H):
    y = dev(wl.rng_for(2, M, H).standard_normal((M, 2 * H)).astype(np.float32))
    gq, gs = Guarded((M, H), torch.int8), Guarded((M,), torch.float32)
    fn(y, gq.t, gs.t)
    gq.check(fn.__name__ + " q")
    gs.check(fn.__name__ + " s_a")
    q, s = fn(y)
    same(gq.t, q, fn.__name__)
    same(gs.t, s, fn.__name__)


@pytest.mark.parametrize("M", [1, 3, 5, 8, 13, 16])
@pytest.mark.parametrize("N,K", [(272, 384), (2064, 2688), (4112, 384)])
def test_gemv_outputs_stay_in_bounds(gpu, M, N, K):
    p, s, x, q, sa = weights(M, N, K)
    g = Guarded((M, N), torch.float32)
    bn.bitnet_w2a8_gemv(p, s, q, sa, N, K, y=g.t)
    g.check(f"gemv {M}x{N}x{K}")
    same(g.t, bn.bitnet_w2a8_gemv(p, s, q, sa, N, K), "gemv")
    ga = Guarded((M, N), torch.int32)
    bn.bitnet_w2a8_acc_i32(p, q, N, K, acc=ga.t)
    ga.check(f"acc {M}x{N}x{K}")
    same(ga.t, bn.bitnet_w2a8_acc_i32(p, q, N, K), "acc")


@pytest.mark.parametrize("M", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("N,K", [(272, 384), (4112, 384), (2560, 1280)])
@pytest.mark.parametrize("junction", [False, "sum", "relu2_glu"])
def test_gemv_act_outputs_stay_in_bounds(gpu, M, N, K, junction):
    p, s, x, q, sa = weights(M, N, K, seed=1)
    if junction:
        x = dev(wl.rng_for(3, M, K).standard_normal((M, 2 * K)).astype(np.float32))
    gy, gq, gs = Guarded((M, N), torch.float32), Guarded((M, K), torch.int8), Guarded((M,), torch.float32)
    bn.bitnet_w2a8_gemv_act(p, s, x, N, K, fold=junction, y=gy.t, q_out=gq.t, s_a_out=gs.t)
    for g, w in ((gy, "y"), (gq, "q_out"), (gs, "s_a_out")):
        g.check(f"gemv_act {junction} {M}x{N}x{K} {w}")
    same(gy.t, bn.bitnet_w2a8_gemv_act(p, s, x, N, K, fold=junction), "gemv_act")


@pytest.mark.parametrize("M,N,K", [(17, 272, 384), (130, 2064, 384), (300, 160, 640), (3207, 2064, 384),
                                   (100, 13824, 640)])
@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float32])
def test_gemm_outputs_stay_in_bounds(gpu, M, N, K, ydt):
    p, s, x, q, sa = weights(M, N, K, seed=2)
    g = Guarded((M, N), ydt)
    bn.bitnet_w2a8_gemm(p, s, q, sa, N, K, y=g.t)
    g.check(f"gemm {M}x{N}x{K} {ydt}")
    same(g.t, bn.bitnet_w2a8_gemm(p, s, q, sa, N, K, out_dtype=ydt), "gemm")
    ga = Guarded((M, N), torch.int32)
    bn.bitnet_w2a8_acc_i32(p, q, N, K, acc=ga.t)
    ga.check(f"acc {M}x{N}x{K}")


@pytest.mark.parametrize("G", [64, 0])
@pytest.mark.parametrize("M,N,K", [(3, 272, 384), (130, 2064, 384), (3207, 2064, 384)])
def test_format_variant_outputs_stay_in_bounds(gpu, G, M, N, K):
    p, s, x, q, sa = weights(M, N, K, seed=3, G=G)
    if M <= 16:
        g = Guarded((M, N), torch.float32)
        bn.bitnet_w2a8_gemv_g(p, s, q, sa, N, K, G, y=g.t)
        g.check(f"gemv_g G={G} {M}x{N}x{K}")
        same(g.t, bn.bitnet_w2a8_gemv_g(p, s, q, sa, N, K, G), "gemv_g")
    for ydt in (torch.bfloat16, torch.float32):
        g = Guarded((M, N), ydt)
        bn.bitnet_w2a8_gemm_g(p, s, q, sa, N, K, G, y=g.t)
        g.check(f"gemm_g G={G} {M}x{N}x{K} {ydt}")
        same(g.t, bn.bitnet_w2a8_gemm_g(p, s, q, sa, N, K, G, out_dtype=ydt), "gemm_g")


@pytest.mark.parametrize("tiles", [1, 2, 4])
@pytest.mark.parametrize("N,K", [(272, 384), (4112, 1280)])
def test_lut_outputs_stay_in_bounds(gpu, tiles, N, K):
    p, s, x, q, sa = weights(1, N, K, seed=4)
    gy, ga = Guarded((1, N), torch.float32), Guarded((1, N), torch.int32)
    bn.bitnet_w2a8_gemv_lut(p, s, q, sa, N, K, tiles, y=gy.t, acc=ga.t)
    gy.check(f"lut y {N}x{K} tiles {tiles}")
    ga.check(f"lut acc {N}x{K} tiles {tiles}")
    y, acc = bn.bitnet_w2a8_gemv_lut(p, s, q, sa, N, K, tiles, with_acc=True)
    same(gy.t, y, "lut y")
    same(ga.t, acc, "lut acc")


@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("junction", ["sum", "relu2_glu"])
def test_chain_output_and_workspace_stay_in_bounds(gpu, M, junction):
    shapes = [(384, 384), (640, 384), (2304, 640), (272, 1152)]  # 17 tiles last, fold 2304 -> 1152
    ws, folds = [], []
    for i, (N, K) in enumerate(shapes):
        c = wl.small_case(60 + i, 1, N, K)
        ws.append(bn.PackedWeight.from_ternary(c.T, (c.S / np.float32(np.sqrt(K))).astype(np.float32)))
        folds.append(junction if i == 3 else False)
    chain = bn.Chain(ws, folds)
    x = dev(wl.normal_act(wl.rng_for(6, M), M, 384).view(np.int16)).view(torch.bfloat16)
    nb = chain.workspace_bytes(M)
    gw = Guarded((nb,), torch.uint8)
    gw.t.fill_(0)
    gy = Guarded((M, shapes[-1][0]), torch.float32)
    st = bn.lib().bitnet_w2a8_chain(ctypes.cast(chain._arr, ctypes.c_void_p), len(ws), ctypes.c_void_p(x.data_ptr()),
                                    bn.BITNET_DT_BF16, M, ctypes.c_void_p(gy.t.data_ptr()),
                                    ctypes.c_void_p(gw.t.data_ptr()), nb,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == bn.BITNET_OK
    gy.check(f"chain y M={M}")
    gw.check(f"chain workspace M={M}")
    same(gy.t, chain(x), "chain")


@pytest.mark.parametrize("M", [1, 3, 8])
def test_static_chain_output_stays_in_bounds(gpu, M):
    """bitnet_w2a8_chain_static writes only its y (its workspace is the library's own array)."""
    shapes = [(384, 384), (640, 384), (2304, 640), (272, 1152)]
    ws = []
    for i, (N, K) in enumerate(shapes):
        c = wl.small_case(70 + i, 1, N, K)
        ws.append(bn.PackedWeight.from_ternary(c.T, (c.S / np.float32(np.sqrt(K))).astype(np.float32)))
    chain = bn.Chain(ws, [False, False, False, "sum"])
    x = dev(wl.normal_act(wl.rng_for(7, M), M, 384).view(np.int16)).view(torch.bfloat16)
    gy = Guarded((M, shapes[-1][0]), torch.float32)
    st = bn.lib().bitnet_w2a8_chain_static(ctypes.cast(chain._arr, ctypes.c_void_p), len(ws),
                                           ctypes.c_void_p(x.data_ptr()), bn.BITNET_DT_BF16, M,
                                           ctypes.c_void_p(gy.t.data_ptr()),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == bn.BITNET_OK
    gy.check(f"static chain y M={M}")
    same(gy.t, chain(x), "static chain")


@pytest.mark.parametrize("junction", ["sum", "relu2_glu"])
def test_persistent_chain_output_and_workspace_stay_in_bounds(gpu, junction):
    """The one-launch chain writes only its y and the prepared size of its workspace."""
    shapes = [(384, 384), (640, 384), (2304, 640), (272, 1152)]  # 17 tiles last, two-half input in front
    ws = []
    for i, (N, K) in enumerate(shapes):
        c = wl.small_case(80 + i, 1, N, K)
        ws.append(bn.PackedWeight.from_ternary(c.T, (c.S / np.float32(np.sqrt(K))).astype(np.float32)))
    chain = bn.Chain(ws, [False, False, False, junction])
    x = dev(wl.normal_act(wl.rng_for(8, 1), 1, 384).view(np.int16)).view(torch.bfloat16)
    plan = chain.plan_persistent(1, bn.BITNET_DT_BF16)
    gw = Guarded((plan.workspace_bytes,), torch.uint8)
    gy = Guarded((1, shapes[-1][0]), torch.float32)
    st = bn.lib().bitnet_w2a8_chain_persistent(plan.table.data_ptr(), plan.n, x.data_ptr(), bn.BITNET_DT_BF16, 1,
                                               gy.t.data_ptr(), gw.t.data_ptr(), plan.workspace_bytes,
                                               torch.cuda.current_stream().cuda_stream)
    assert st == bn.BITNET_OK
    gy.check(f"persistent chain y ({junction})")
    gw.check(f"persistent chain workspace ({junction})")
    assert int(gw.t[:4].view(torch.int32).item()) == 0  # status: every wait succeeded
    same(gy.t, chain.persistent(x), "persistent chain")
