"""The decode stack the benchmark times, checked whole: 48 independently
seeded layers (hidden 2048, 128 experts, top-8, intermediate 768, Q8_0,
fp32 activations), one token, one moe_decode_layer call per layer, captured
as one HIP graph and replayed, every layer's routing and output compared
with the oracle."""
import numpy as np
import pytest
import torch

from expert_offload_amd import layer
from gen import inputs as gi
import oracle

from gpu_util import DEV, check_routed_layer, note
import expert_offload_amd as moe

pytestmark = pytest.mark.gpu

DECODE_TOL = 1e-3
MARGIN = 1e-3  # experts whose oracle logit is this close to the k-th are made resident too


def test_decode_stack_all_layers_graph():
    wl = gi.workload("decode_q8_0_h2048_e128")
    T = 1
    x = gi.activations(wl, T)
    routers = [gi.router_weight(wl, l) for l in range(wl.layers)]
    # experts each layer can route to: the oracle's top k plus any within MARGIN of the k-th logit
    needed = []
    for l in range(wl.layers):
        lo = oracle.router_logits(x, routers[l])[0]
        kth = np.sort(lo)[::-1][wl.k - 1]
        needed += [(l, int(e)) for e in np.nonzero(lo >= kth - MARGIN)[0]]
    note(f"decode stack: {wl.layers} layers, {len(needed)} resident experts")
    slot_of = {key: i for i, key in enumerate(needed)}
    pool = layer.SlotPool(wl.qtype, wl.H, wl.I, len(needed), device=DEV)
    blocks = {}

    def put(l, e, b):
        blocks[(l, e)] = b
        pool.put(slot_of[(l, e)], layer.pack_expert(wl.qtype, wl.H, wl.I, *b))

    gi.generate_blocks_parallel(wl, needed, put)
    tables = []
    for l in range(wl.layers):
        t = np.full(wl.E, -1, dtype=np.int32)  # a route to any other expert gives NaN and an error
        for (ll, e), s in slot_of.items():
            if ll == l:
                t[e] = s
        tables.append(torch.from_numpy(t).to(DEV))
    ctx = moe.Ctx(0)
    xd = torch.from_numpy(x).to(DEV)
    wr = [torch.from_numpy(r).to(DEV) for r in routers]
    bufs = [layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV) for _ in range(wl.layers)]

    def run():
        for l in range(wl.layers):
            layer.forward(ctx, bufs[l], pool.base(), pool.slot_bytes, pool.n_slots, tables[l], xd,
                          router_w=wr[l], fused="layer")

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    refs, getters = [], []
    for l in range(wl.layers):
        def get(e, l=l):
            return blocks[(l, e)]
        getters.append(get)
        refs.append(oracle.moe_layer(x, wl.qtype, get, wl.k, router_w=routers[l]))
    for rep in range(2):
        for b in bufs:
            for name in ("logits", "w", "y", "out"):
                getattr(b, name).fill_(float("nan"))
            b.ids.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        moe.moe_ctx_check(ctx)
        note(f"   graph replay {rep}: checking {wl.layers} layers")
        for l in range(wl.layers):
            b, get = bufs[l], getters[l]
            check_routed_layer(b.ids.cpu().numpy(), b.w.cpu().numpy(), b.logits.cpu().numpy(), b.y.cpu().numpy(),
                               b.out.cpu().numpy(), refs[l], DECODE_TOL, T,
                               lambda lo, get=get: oracle.moe_layer(x, wl.qtype, get, wl.k, logits=lo))
    ctx.close()
