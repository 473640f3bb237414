"""GPU parity of the one-launch (persistent) decode chain, bitnet_w2a8_chain_persistent.

Every layer's output stays in the workspace after the launch, so each product is
checked element by element against the oracle fed the GPU's own input to it (the
layer-local parity of the launch-per-layer chain), and each requantisation against the
oracle's own decision (R11 with identical inputs).  Also: graph capture and replay, and
the bounded waits giving up when the host withholds a layer's output (every kernel still
ends)."""
import numpy as np
import pytest

import bit_gemv_i2_amd as bn
import oracle
import oracle_pool as op
import parity_stats
import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# (N, K, junction in front); K of a layer behind a junction is half the previous N
SMALL = [(256, 512, False), (384, 256, False), (1024, 384, False), (384, 512, True), (2304, 384, False),
         (272, 1152, True)]


def _chain(seed, junction):
    ws, Ts, Ss = [], [], []
    for i, (N, K, f) in enumerate(SMALL):
        r = wl.rng_for(81, seed, i)
        T = wl.ternary_uniform(r, N, K)
        S = wl.uniform_scales(r, N, K, div=np.sqrt(7 * K / 6))
        Ts.append(T)
        Ss.append(S)
        ws.append(bn.PackedWeight.from_ternary(T, S))
    return bn.Chain(ws, [junction if f else False for (_, _, f) in SMALL]), Ts, Ss


def _x(K, seed, xdt):
    xb = wl.normal_act(wl.rng_for(82, seed), 1, K)
    if xdt == "bf16":
        return xb, torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    x = wl.bf16_to_f32(xb) * np.float32(0.75)
    return x, torch.from_numpy(x).cuda()


def _check_layers(chain, Ts, Ss, junction, xin, xdt, outs, y):
    prev = None
    for k, (N, K, f) in enumerate(SMALL):
        if k == 0:
            q, s = oracle.quant_act_bf16(xin) if xdt == "bf16" else oracle.quant_act_f32(xin)
        elif f:
            q, s = oracle.fold_quant(prev) if junction == "sum" else oracle.glu_quant(prev)
        else:
            q, s = oracle.quant_act_f32(prev)
        ref = oracle.w2a8(oracle.pack_i2s(Ts[k]), Ss[k], q, s, N, K)
        got = outs[k] if k < len(SMALL) - 1 else y
        parity_stats.record(got, ref["y64"], ref["mag"])
        ratio, bad, _ = op.f32_check(got, ref["y64"], ref["mag"])
        assert bad == 0, f"layer {k}: {bad} outputs outside the tolerance (worst {ratio:.3g}x)"
        prev = got


@pytest.mark.parametrize("xdt", ["bf16", "f32"])
@pytest.mark.parametrize("junction", ["sum", "relu2_glu"])
def test_persistent_chain_every_layer_against_the_oracle(gpu, junction, xdt):
    chain, Ts, Ss = _chain(1, junction)
    xin, x = _x(SMALL[0][1], 2, xdt)
    y = chain.persistent(x)
    torch.cuda.synchronize()
    bxdt = bn.BITNET_DT_BF16 if xdt == "bf16" else bn.BITNET_DT_F32
    outs, status = chain.persistent_layer_outputs(1, bxdt)
    assert status == 0
    _check_layers(chain, Ts, Ss, junction, xin, xdt, outs, y.cpu().numpy())
    # a second call on the same workspace (refilled before the launch) gives the same result
    y2 = chain.persistent(x)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))


def test_persistent_chain_with_a_caller_workspace(gpu):
    """A workspace the caller passes serves the launch and the read-back of the layer
    outputs; the results equal those of the binding's own workspace bit for bit."""
    chain, Ts, Ss = _chain(4, "relu2_glu")
    xin, x = _x(SMALL[0][1], 5, "f32")
    with pytest.raises(ValueError):
        chain.persistent_layer_outputs(1, bn.BITNET_DT_F32)  # no call with the binding's workspace yet
    plan = chain.plan_persistent(1, bn.BITNET_DT_F32)
    mine = torch.empty(plan.workspace_bytes + 4096, dtype=torch.uint8, device="cuda")
    y1 = chain.persistent(x, workspace=mine)
    torch.cuda.synchronize()
    outs1, st1 = chain.persistent_layer_outputs(1, bn.BITNET_DT_F32, workspace=mine)
    assert st1 == 0
    _check_layers(chain, Ts, Ss, "relu2_glu", xin, "f32", outs1, y1.cpu().numpy())
    y2 = chain.persistent(x)
    torch.cuda.synchronize()
    outs2, st2 = chain.persistent_layer_outputs(1, bn.BITNET_DT_F32)
    assert st2 == 0
    assert np.array_equal(y1.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))
    for a, b in zip(outs1, outs2):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    with pytest.raises(ValueError):
        chain.persistent_layer_outputs(1, bn.BITNET_DT_F32, workspace=mine[:16])


def test_persistent_chain_graph_replays(gpu):
    chain, Ts, Ss = _chain(3, "sum")
    K0 = SMALL[0][1]
    xs = [_x(K0, 10 + i, "bf16")[1] for i in range(4)]
    eager = []
    for x in xs:
        eager.append(chain.persistent(x).cpu().numpy())
    xbuf = torch.empty_like(xs[0])
    ybuf = torch.empty((1, SMALL[-1][0]), dtype=torch.float32, device="cuda")
    xbuf.copy_(xs[0])
    chain.persistent(xbuf, y=ybuf)  # plan, table and workspace exist before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain.persistent(xbuf, y=ybuf)
    for i, x in enumerate(xs):
        xbuf.copy_(x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(ybuf.cpu().numpy().view(np.uint32), eager[i].view(np.uint32)), f"replay {i}"
        assert chain.persistent_layer_outputs(1, bn.BITNET_DT_BF16)[1] == 0


def test_persistent_chain_bounded_wait_gives_up(gpu):
    """The host withholds layer 2's output (test-only knob) and sets a tiny spin limit:
    the workgroups waiting for it give up, record the layer in the status word and end;
    the launch completes.  A normal launch afterwards is correct again."""
    chain, Ts, Ss = _chain(5, "sum")
    xin, x = _x(SMALL[0][1], 6, "bf16")
    chain.persistent(x, spin_limit=64, withhold=2)
    torch.cuda.synchronize()
    _, status = chain.persistent_layer_outputs(1, bn.BITNET_DT_BF16)
    assert status >= 4, status  # layer 3 (or a later one) gave up: status = its index + 1
    y = chain.persistent(x)
    torch.cuda.synchronize()
    outs, status = chain.persistent_layer_outputs(1, bn.BITNET_DT_BF16)
    assert status == 0
    _check_layers(chain, Ts, Ss, "sum", xin, "bf16", outs, y.cpu().numpy())


def test_persistent_chain_stops_on_a_table_that_does_not_fit_the_workspace(gpu):
    """The caller declares a workspace 4 bytes short of the plan (the buffer itself is
    whole, so nothing could land outside it): every workgroup stops at the first layer
    whose output would not fit, the status word says which (negative), nothing past the
    declared size is written, and the launch ends."""
    chain, _, _ = _chain(9, "sum")
    _, x = _x(SMALL[0][1], 10, "bf16")
    plan = chain.plan_persistent(1, bn.BITNET_DT_BF16)
    ws = torch.full((plan.workspace_bytes + 256,), 0x5A, dtype=torch.uint8, device="cuda")
    y = torch.zeros((1, SMALL[-1][0]), dtype=torch.float32, device="cuda")
    short = plan.workspace_bytes - 4
    st = bn.lib().bitnet_w2a8_chain_persistent(plan.table.data_ptr(), plan.n, x.data_ptr(), bn.BITNET_DT_BF16, 1,
                                               y.data_ptr(), ws.data_ptr(), short,
                                               torch.cuda.current_stream().cuda_stream)
    assert st == bn.BITNET_OK
    torch.cuda.synchronize()
    host = ws.cpu().numpy()
    # the last intermediate output (layer n - 2) ends exactly at the plan's size
    assert int(host[:4].view(np.int32)[0]) == -(plan.n - 1)
    assert (host[short:] == 0x5A).all()
    assert (y.cpu().numpy() == 0).all()


def test_persistent_chain_rejects_batches_above_one(gpu):
    chain, _, _ = _chain(7, "sum")
    x = torch.zeros((2, SMALL[0][1]), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bn.BitnetError) as ei:
        chain.persistent(x)
    assert ei.value.status == bn.BITNET_ERR_UNSUPPORTED_SHAPE


@pytest.mark.slow
@pytest.mark.parametrize("junction", ["sum", "relu2_glu"])
def test_persistent_stack_30_layers_every_product(gpu, junction):
    """The 30-layer stack in one launch at batch 1: all 180 products element by element
    against the oracle fed the GPU's own input, and the requantisation decisions."""
    ws = []
    for layer in range(wl.STACK_LAYERS):
        for idx in range(6):
            T, S = wl.stack_matrix(layer, idx)
            ws.append(bn.PackedWeight.from_ternary(T, S))
    n = len(ws)
    chain = bn.Chain(ws, [junction if i % 6 == 5 else False for i in range(n)])
    xb = wl.stack_input(1)
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    y = chain.persistent(x)
    torch.cuda.synchronize()
    outs, status = chain.persistent_layer_outputs(1, bn.BITNET_DT_BF16)
    assert status == 0
    outs = outs + [y.cpu().numpy()]
    tasks = []
    for p in range(n):
        layer, idx = divmod(p, 6)
        kind = "bf16" if p == 0 else (junction if idx == 5 else "plain")
        nxt = None if p == n - 1 else (junction if idx == 4 else "plain")
        tasks.append((p, layer, idx, kind, nxt, [(1, xb if p == 0 else outs[p - 1], outs[p])]))
    print(f"persistent stack {junction}: oracle on {n} products in {op.workers()} processes", flush=True)
    with op.pool() as ex:
        res = [r for chunk in ex.map(op.stack_product, tasks, chunksize=3) for r in chunk]
    assert len(res) == n
    codes = sum(r["codes"] for r in res)
    flips = sum(r["n_diff"] for r in res)
    print(f"persistent stack {junction}: worst error / bound {max(r['ratio'] for r in res):.3f}, plain max "
          f"relative error {max(r['plain_rel'] for r in res):.3e}, requantisation codes at a midpoint that "
          f"differ {flips} of {codes}", flush=True)
    parity_stats.note(f"persistent stack {junction}", max(r["ratio"] for r in res), max(r["plain_rel"] for r in res))
    for r in res:
        where = f"{junction} product {r['p']}"
        assert r["bad"] == 0, f"{where}: {r['bad']} outputs outside the tolerance (worst {r['ratio']:.3g}x)"
        assert r["unjustified"] == 0 and r["max_dq"] <= 1, where
        assert r["n_diff"] <= max(1, r["codes"] // 1000), where


def _plan_fields(shapes, folds, xdt):
    """The persistent plan of a chain on this device (layer addresses are not read)."""
    import ctypes
    n = len(shapes)
    arr = (bn.ChainLayer * n)()
    for i, ((N, K), f) in enumerate(zip(shapes, folds)):
        arr[i] = bn.ChainLayer(0x100000, 0x200000, N, K, f)
    nb = bn.lib().bitnet_w2a8_persist_table_bytes(n)
    host = np.zeros(nb, np.uint8)
    ws = ctypes.c_size_t(0)
    st = bn.lib().bitnet_w2a8_persist_prepare(ctypes.cast(arr, ctypes.c_void_p), n, 1, xdt, 0,
                                               host.ctypes.data_as(ctypes.c_void_p), nb, ctypes.byref(ws))
    return st, host.view(np.int32).reshape(n, 16)


def _random_chain_spec(seed, xdt):
    """A random chain the device can run in one launch: K up to 16384 (8192 behind a
    junction), so that 4, 2 and 1 row tiles per workgroup all occur."""
    r = wl.rng_for(84, seed)
    while True:
        n = int(r.integers(3, 7))
        shapes, folds = [], []
        K, fold = 128 * int(r.integers(1, 41)), 0
        for i in range(n):
            last = i == n - 1
            N = 16 * int(r.integers(1, 200)) if last else 128 * int(r.integers(1, 129))
            shapes.append((N, K))
            folds.append(fold)
            if not last:
                fold = int(r.integers(0, 3)) if (N % 256 == 0 and N // 2 <= 8192) else 0
                K = N // 2 if fold else N
        st, t = _plan_fields(shapes, folds, xdt)
        if st == bn.BITNET_OK:
            return shapes, folds, sorted({int(row[11]) for row in t})


@pytest.mark.parametrize("seed", range(4))
def test_persistent_random_chains_against_the_oracle(gpu, seed):
    """Seeded random chains (shapes, junctions, input type) in one persistent launch: every
    layer's output element by element against the oracle fed the GPU's own input."""
    xdt = "bf16" if seed % 2 == 0 else "f32"
    bxdt = bn.BITNET_DT_BF16 if xdt == "bf16" else bn.BITNET_DT_F32
    shapes, folds, tiles = _random_chain_spec(seed, bxdt)
    print(f"seed {seed}: {xdt} input, layers {shapes}, junctions {folds}, row tiles per workgroup {tiles}",
          flush=True)
    Ts, Ss, ws = [], [], []
    for i, (N, K) in enumerate(shapes):
        r = wl.rng_for(85, seed, i)
        T = wl.ternary_uniform(r, N, K)
        S = wl.uniform_scales(r, N, K, div=np.sqrt(7 * K / 6))
        Ts.append(T)
        Ss.append(S)
        ws.append(bn.PackedWeight.from_ternary(T, S))
    codes = {0: False, 1: "sum", 2: "relu2_glu"}
    chain = bn.Chain(ws, [codes[f] for f in folds])
    xin, x = _x(shapes[0][1], 86 + seed, xdt)
    y = chain.persistent(x)
    torch.cuda.synchronize()
    outs, status = chain.persistent_layer_outputs(1, bxdt)
    assert status == 0
    prev = None
    for k, ((N, K), f) in enumerate(zip(shapes, folds)):
        if k == 0:
            q, s = oracle.quant_act_bf16(xin) if xdt == "bf16" else oracle.quant_act_f32(xin)
        elif f == 1:
            q, s = oracle.fold_quant(prev)
        elif f == 2:
            q, s = oracle.glu_quant(prev)
        else:
            q, s = oracle.quant_act_f32(prev)
        ref = oracle.w2a8(oracle.pack_i2s(Ts[k]), Ss[k], q, s, N, K)
        got = outs[k] if k < len(shapes) - 1 else y.cpu().numpy()
        parity_stats.record(got, ref["y64"], ref["mag"])
        ratio, bad, _ = op.f32_check(got, ref["y64"], ref["mag"])
        assert bad == 0, f"seed {seed} layer {k} ({N}x{K}): {bad} outputs outside the tolerance (worst {ratio:.3g}x)"
        prev = got


def test_persistent_random_chains_cover_every_geometry(gpu):
    """The seeds above between them put 4, 2 and 1 row tiles on a workgroup."""
    seen = set()
    for seed in range(4):
        bxdt = bn.BITNET_DT_BF16 if seed % 2 == 0 else bn.BITNET_DT_F32
        seen |= set(_random_chain_spec(seed, bxdt)[2])
    assert seen == {1, 2, 4}, seen
