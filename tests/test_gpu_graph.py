"""Captured HIP graphs give the same results as eager calls.

The benchmark times every path as replays of a captured graph.  Each test here
captures one path on fixed buffers, then, round after round, writes new seeded
activations into the captured input buffer eagerly, runs the same calls eagerly
into separate outputs, synchronises, replays the graph, and requires the
replay's outputs to equal the eager ones bit for bit (the kernels are
deterministic for a given shape and device)."""
import numpy as np
import pytest

import bit_gemv_i2_amd as bn
import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
ROUNDS = 4


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def bf16_input(seed, M, K):
    return dev(wl.normal_act(wl.rng_for(93, seed), M, K).view(np.int16)).view(torch.bfloat16)


def weights(seed, N, K):
    r = wl.rng_for(91, seed)
    return bn.PackedWeight.from_ternary(wl.ternary_uniform(r, N, K), wl.uniform_scales(r, N, K))


def bits(t):
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16) if t.element_size() == 2 else t


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def check_replays(x, make_input, graph_fn, eager_fn, graph_outs):
    g = capture(graph_fn)
    for r in range(ROUNDS):
        x.copy_(make_input(r))
        want = [t.clone() for t in eager_fn()]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, exp in zip(graph_outs, want):
            assert torch.equal(bits(got), bits(exp)), f"replay {r} differs from the eager result"


@pytest.mark.parametrize("N,K", [(13824, 2560), (2560, 2560)])
def test_fused_step_graph(gpu, N, K):
    w = weights(1, N, K)
    x = bf16_input(100, 1, K)
    y_g = torch.empty((1, N), dtype=torch.float32, device="cuda")
    y_e = torch.empty_like(y_g)
    check_replays(x, lambda r: bf16_input(101 + r, 1, K),
                  lambda: bn.bitnet_w2a8_gemv_act(w.packed, w.scales, x, N, K, y=y_g),
                  lambda: [bn.bitnet_w2a8_gemv_act(w.packed, w.scales, x, N, K, y=y_e)], [y_g])


def test_two_launch_step_graph_8_tokens(gpu):
    N, K, M = 13824, 2560, 8
    w = weights(2, N, K)
    x = bf16_input(200, M, K)
    q_g = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s_g = torch.empty((M,), dtype=torch.float32, device="cuda")
    y_g = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def graph_fn():
        bn.bitnet_quant_act(x, q_g, s_g)
        bn.bitnet_w2a8_gemv(w.packed, w.scales, q_g, s_g, N, K, y=y_g)

    def eager_fn():
        q, s = bn.bitnet_quant_act(x)
        return [q, s, bn.bitnet_w2a8_gemv(w.packed, w.scales, q, s, N, K)]

    check_replays(x, lambda r: bf16_input(201 + r, M, K), graph_fn, eager_fn, [q_g, s_g, y_g])


def test_prefill_graph(gpu):
    N, K, M = 4096, 2560, 200
    w = weights(3, N, K)
    x = bf16_input(300, M, K)
    q_g = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s_g = torch.empty((M,), dtype=torch.float32, device="cuda")
    y_g = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def graph_fn():
        bn.bitnet_quant_act(x, q_g, s_g)
        bn.bitnet_w2a8_gemm(w.packed, w.scales, q_g, s_g, N, K, y=y_g)

    def eager_fn():
        q, s = bn.bitnet_quant_act(x)
        return [bn.bitnet_w2a8_gemm(w.packed, w.scales, q, s, N, K)]

    check_replays(x, lambda r: bf16_input(301 + r, M, K), graph_fn, eager_fn, [y_g])


@pytest.mark.parametrize("M", [1, 8])
def test_chain_graph(gpu, M):
    # 2560 -> 2560 -> 13824 -> (gated junction) 6912 -> 2560: one layer of each stack shape
    shapes = [(2560, 2560, False), (13824, 2560, False), (2560, 6912, "relu2_glu"), (2560, 2560, False)]
    ws = []
    for i, (N, K, _) in enumerate(shapes):
        r = wl.rng_for(95, i)
        ws.append(bn.PackedWeight.from_ternary(wl.ternary_uniform(r, N, K),
                                               wl.uniform_scales(r, N, K, div=np.sqrt(7 * K / 6))))
    chain = bn.Chain(ws, [f for (_, _, f) in shapes])
    x = bf16_input(400 + M, M, 2560)
    y_g = torch.empty((M, 2560), dtype=torch.float32, device="cuda")
    y_e = torch.empty_like(y_g)
    check_replays(x, lambda r: bf16_input(401 + M + r, M, 2560), lambda: chain(x, y=y_g),
                  lambda: [chain(x, y=y_e)], [y_g])
