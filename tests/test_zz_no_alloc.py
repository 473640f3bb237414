"""bitnet_w2a8_chain_static: the decode chain with its workspace in the library's
per-GPU array, for callers that cannot allocate.  Called through the C ABI, it must
give exactly what bitnet_w2a8_chain gives with a caller workspace, on consecutive
calls whose inputs shrink (the array keeps the previous call's contents), and it must
reject a chain whose workspace exceeds the array."""
import ctypes

import numpy as np
import pytest

import bit_gemv_i2_amd as bn
import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _chain(shapes, folds, seed):
    ws = []
    for i, (N, K) in enumerate(shapes):
        c = wl.small_case(seed + i, 1, N, K)
        ws.append(bn.PackedWeight.from_ternary(c.T, (c.S / np.float32(np.sqrt(7 * K / 6))).astype(np.float32)))
    return bn.Chain(ws, folds)


def _x(M, K, seed):
    return torch.from_numpy(wl.normal_act(wl.rng_for(seed, M, K), M, K).view(np.int16)).cuda().view(torch.bfloat16)


def _static(chain, x, y):
    st = bn.lib().bitnet_w2a8_chain_static(ctypes.cast(chain._arr, ctypes.c_void_p), len(chain.weights),
                                            ctypes.c_void_p(x.data_ptr()), bn.BITNET_DT_BF16, x.shape[0],
                                            ctypes.c_void_p(y.data_ptr()),
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_static_chain_matches_workspace_chain_on_shrinking_calls(gpu):
    assert bn.bitnet_w2a8_chain_static_max_bytes() == 4 << 20
    big = _chain([(2560, 2560), (13824, 2560), (2560, 6912), (2560, 2560)], [False, False, "sum", False], 900)
    small = _chain([(384, 640), (1024, 384), (272, 512)], [False, False, "relu2_glu"], 910)
    # first call: the full stack shapes at 8 tokens; second: a smaller chain at 3 tokens, then 1
    for chain, M, K, seed in [(big, 8, 2560, 1), (small, 3, 640, 2), (small, 1, 640, 3), (big, 2, 2560, 4)]:
        x = _x(M, K, seed)
        y = torch.full((M, chain.weights[-1].N), float("nan"), dtype=torch.float32, device="cuda")
        assert _static(chain, x, y) == bn.BITNET_OK
        ref = chain(x)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32)), (M, K)
        # the binding's wrapper of the same entry point
        y2 = chain.call_static(x)
        torch.cuda.synchronize()
        assert np.array_equal(y2.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))


def test_static_chain_rejects_a_workspace_beyond_the_array(gpu):
    # 16 tokens x 262144-wide activations need 2 x 16 MiB: more than the 4 MiB array
    wide = _chain([(262144, 128)], [False], 920)
    assert wide.workspace_bytes(16) > bn.bitnet_w2a8_chain_static_max_bytes()
    x = _x(16, 128, 5)
    y = torch.zeros((16, 262144), dtype=torch.float32, device="cuda")
    assert _static(wide, x, y) == bn.BITNET_ERR_UNSUPPORTED_SHAPE
    assert np.all(y.cpu().numpy() == 0)
