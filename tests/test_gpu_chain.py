"""GPU parity of the chained decode (a stack of W2A8 layers with per-token
requantisation and the gate+up fold between them).

Layer-local: every layer of the chain is compared with the oracle fed the
GPU's own input to that layer (bit-exact int8 / factors, fp32 within the
product tolerance).  The chain equals the products called one by one, bit for
bit.  The full 30-layer stack at its real shapes is checked product by product
in test_gpu_stack_full.py."""
import ctypes

import numpy as np
import pytest

import bit_gemv_i2_amd as bn
import oracle
import parity_stats
import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
RTOL = 1e-5


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# (N, K, junction in front): K of a layer behind a junction is half the previous N
SMALL = [(256, 512, False), (384, 256, False), (1024, 384, False), (384, 512, True), (128, 384, False)]
JUNCTIONS = ["sum", "relu2_glu"]


def _small_chain(seed, junction="sum"):
    Ts, Ss, ws = [], [], []
    for i, (N, K, f) in enumerate(SMALL):
        r = wl.rng_for(71, seed, i)
        T = wl.ternary_uniform(r, N, K)
        S = wl.uniform_scales(r, N, K, div=np.sqrt(7 * K / 6))
        Ts.append(T)
        Ss.append(S)
        ws.append(bn.PackedWeight.from_ternary(T, S))
    return Ts, Ss, ws, [junction if f else False for (_, _, f) in SMALL]


def _oracle_junction(junction, prev):
    return oracle.fold_quant(prev) if junction == "sum" else oracle.glu_quant(prev)


@pytest.mark.parametrize("junction", JUNCTIONS)
@pytest.mark.parametrize("M", [1, 3, 8])
def test_chain_layer_local_parity(gpu, M, junction):
    Ts, Ss, ws, folds = _small_chain(M, junction)
    xb = wl.normal_act(wl.rng_for(72, M), M, SMALL[0][1])
    x = dev(xb.view(np.int16)).view(torch.bfloat16)
    prev = None
    for k in range(len(SMALL)):
        y = host(bn.Chain(ws[:k + 1], folds[:k + 1])(x))
        if k == 0:
            q, s = oracle.quant_act_bf16(xb)
        elif folds[k]:
            q, s = _oracle_junction(folds[k], prev)
        else:
            q, s = oracle.quant_act_f32(prev)
        N, K, _ = SMALL[k]
        ref = oracle.w2a8(oracle.pack_i2s(Ts[k]), Ss[k], q, s, N, K)
        parity_stats.record(y, ref["y64"], ref["mag"])
        bound = RTOL * np.maximum(np.abs(ref["y64"]), ref["mag"])
        assert np.all(np.abs(y.astype(np.float64) - ref["y64"]) <= bound), f"layer {k}"
        prev = y


@pytest.mark.parametrize("junction", JUNCTIONS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
def test_chain_equals_products_called_one_by_one(gpu, M, junction):
    Ts, Ss, ws, folds = _small_chain(10 + M, junction)
    xb = wl.normal_act(wl.rng_for(73, M), M, SMALL[0][1])
    x = dev(xb.view(np.int16)).view(torch.bfloat16)
    y_chain = host(bn.Chain(ws, folds)(x))
    h = x
    for w, f in zip(ws, folds):
        if M <= 4:
            h = bn.bitnet_w2a8_gemv_act(w.packed, w.scales, h, w.N, w.K, fold=f)
        else:
            if f == "sum":
                q, s = bn.bitnet_quant_act_fold(h)
            elif f:
                q, s = bn.bitnet_quant_act_relu2_glu(h)
            else:
                q, s = bn.bitnet_quant_act(h)
            h = bn.bitnet_w2a8_gemv(w.packed, w.scales, q, s, w.N, w.K)
    assert np.array_equal(y_chain.view(np.uint32), host(h).view(np.uint32))


def test_chain_rejects_mismatched_shapes(gpu):
    Ts, Ss, ws, folds = _small_chain(3)
    x = torch.zeros((1, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bn.BitnetError):
        bn.Chain([ws[0], ws[2]], [False, False])(x)      # K of layer 1 != N of layer 0
    with pytest.raises(bn.BitnetError):
        bn.Chain(ws[:4], [False, False, False, False])(x)  # the fold is missing
    with pytest.raises(bn.BitnetError):
        bn.Chain(ws[:1], [True])(x)                        # layer 0 cannot fold
    # no such junction: the C entry point rejects it before any launch
    good = bn.Chain(ws[:4], [False, False, False, "sum"])
    ws_buf = good.workspace(1)
    y = torch.empty((1, ws[3].N), dtype=torch.float32, device="cuda")
    good._arr[3].fold_input = 3
    st = bn.lib().bitnet_w2a8_chain(ctypes.cast(good._arr, ctypes.c_void_p), 4, x.data_ptr(), bn.BITNET_DT_BF16, 1,
                                    y.data_ptr(), ws_buf.data_ptr(), ws_buf.numel(), None)
    assert st == bn.BITNET_ERR_INVALID_ARG
    assert bn.lib().bitnet_w2a8_chain_workspace_bytes(ctypes.cast(good._arr, ctypes.c_void_p), 4, 1) == 0
