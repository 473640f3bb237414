"""Full-size parity of the decode stack: 30 layers of 4 x (2560x2560), 13824x2560
and 2560x6912 W2A8 products (a ~2.4B-parameter ternary model's linear layers,
[P3] "Why WASM"), run by bitnet_w2a8_chain with the linear fold or the squared-ReLU
gate in front of each 2560x6912 product ([P4] "Architecture-specific SIMD
acceleration"), at batch 1, 2, 4 and 8 -- every fused and two-launch form the chain
chooses between.

Element by element at every one of the 180 products (layer-local: the oracle is fed
the GPU's own input to that product):
  * y within 1e-5 * max(|y|, mag) of the oracle's exact value;
  * the requantisation decisions for the next product (R11 with identical inputs): the
    oracle quantises the GPU's fp32 output and its own fp32 output of the same
    product; codes may differ only where the exact value sits within the fp32 error
    band of a rounding midpoint, by exactly one, and in at most 1e-3 of the codes.
A free-running comparison (oracle and GPU each on their own previous outputs) is not a
valid acceptance test past the first such midpoint: one flipped code moves every
output of the next product by about one part in 10^4, which flips further codes, and
within two layers the two valid evaluations disagree in most codes.  The first product
at which the free-running chains part is therefore reported, not asserted.

The GPU outputs of every product inside the chain come from running the chain on each
prefix of the layer list: each layer's launch form depends only on that layer and the
batch, so a prefix computes exactly the values the whole chain computes there."""
import numpy as np
import pytest

import bit_gemv_i2_amd as bn
import oracle_pool as op
import parity_stats
import workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
torch = pytest.importorskip("torch")

BATCHES = (1, 2, 4, 8)
JUNCTIONS = ("sum", "relu2_glu")


@pytest.fixture(scope="module")
def stack(gpu):
    ws = []
    for layer in range(wl.STACK_LAYERS):
        for idx in range(6):
            T, S = wl.stack_matrix(layer, idx)
            ws.append(bn.PackedWeight.from_ternary(T, S))
    yield ws
    del ws
    torch.cuda.empty_cache()


def chain_outputs(ws, folds, x):
    """The output of every product of the chain, from the chain run on each prefix."""
    outs = [bn.Chain(ws[:k + 1], folds[:k + 1])(x) for k in range(len(ws))]
    full = bn.Chain(ws, folds)(x)
    torch.cuda.synchronize()
    host = [o.cpu().numpy() for o in outs]
    assert np.array_equal(full.cpu().numpy().view(np.uint32), host[-1].view(np.uint32))
    return host


@pytest.mark.parametrize("junction", JUNCTIONS)
def test_stack_30_layers_every_product_element_wise(gpu, stack, junction):
    n = len(stack)
    folds = [junction if i % 6 == 5 else False for i in range(n)]
    runs = {}
    for M in BATCHES:
        xb = wl.stack_input(M)
        print(f"stack {junction} M={M}: running {n} prefix chains", flush=True)
        x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        runs[M] = (xb, chain_outputs(stack, folds, x))
    tasks = []
    for p in range(n):
        layer, idx = divmod(p, 6)
        kind = "bf16" if p == 0 else (junction if idx == 5 else "plain")
        nxt = None if p == n - 1 else (junction if idx == 4 else "plain")
        tasks.append((p, layer, idx, kind, nxt,
                      [(M, xb if p == 0 else outs[p - 1], outs[p]) for M, (xb, outs) in runs.items()]))
    print(f"stack {junction}: oracle on {n} products x batches {BATCHES} in {op.workers()} processes", flush=True)
    with op.pool() as ex:
        res = [r for chunk in ex.map(op.stack_product, tasks, chunksize=3) for r in chunk]
    assert len(res) == n * len(BATCHES)
    for M in BATCHES:
        rows = sorted((r for r in res if r["M"] == M), key=lambda r: r["p"])
        codes = sum(r["codes"] for r in rows)
        flips = sum(r["n_diff"] for r in rows)
        first = next((r["p"] for r in rows if r["n_diff"]), None)
        print(f"stack {junction} M={M}: worst error / bound {max(r['ratio'] for r in rows):.3f}, plain max relative "
              f"error {max(r['plain_rel'] for r in rows):.3e}, requantisation codes at a midpoint that differ "
              f"{flips} of {codes}; free-running chains first part at product "
              f"{'none' if first is None else first}", flush=True)
        parity_stats.note(f"stack {junction} M={M}", max(r["ratio"] for r in rows), max(r["plain_rel"] for r in rows))
        for r in rows:
            where = f"{junction} M={M} product {r['p']} (layer {r['p'] // 6}, matrix {r['p'] % 6})"
            assert r["bad"] == 0, f"{where}: {r['bad']} outputs outside the tolerance (worst {r['ratio']:.3g}x)"
            assert r["unjustified"] == 0, f"{where}: {r['unjustified']} codes differ away from a rounding midpoint"
            assert r["max_dq"] <= 1, f"{where}: a code differs by {r['max_dq']}"
            assert r["n_diff"] <= max(1, r["codes"] // 1000), f"{where}: {r['n_diff']} of {r['codes']} codes differ"
        assert flips <= codes // 1000
