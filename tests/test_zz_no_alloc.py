"""moe_decode_layer_static (the decode layer with its workspace in the
library's static device array, for callers that cannot allocate) through
the C ABI, against moe_decode_layer on the same inputs: bit-identical
routing results and outputs on two calls in a row, the second smaller than
the first; replays of a HIP graph that captured it; and the host-side
refusal of a batch whose workspace exceeds the array."""
import numpy as np
import pytest
import torch

import expert_offload_amd as moe
from expert_offload_amd import _lib as L
from expert_offload_amd import layer
from gen import inputs as gi
import oracle

from gpu_util import DEV, ResidentLayer, check_routed_layer, dev, note

pytestmark = pytest.mark.gpu

KEYS = ("logits", "ids", "w", "offsets", "sorted_pairs", "pair_pos", "active", "y", "out")


@pytest.fixture(scope="module")
def ctx():
    c = moe.Ctx(0)
    yield c
    c.close()


@pytest.fixture(scope="module")
def decode_layer():
    return ResidentLayer(gi.workload("decode_q8_0_h2048_e128"), layer_idx=0)


def _poisoned(wl, T):
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV)
    for name in ("logits", "w", "y", "out"):
        getattr(buf, name).fill_(float("nan"))
    for name in ("ids", "offsets", "sorted_pairs", "pair_pos", "active"):
        getattr(buf, name).fill_(-7)
    return buf


def _run(ctx, rl, T, x, wr, fused, buf=None, stream=None):
    wl = rl.wl
    buf = buf or _poisoned(wl, T)
    layer.forward(ctx, buf, rl.pool.base(), rl.pool.slot_bytes, rl.pool.n_slots, rl.slot_table, x,
                  router_w=wr, fused=fused, stream=stream)
    return buf


def _read(buf):
    torch.cuda.synchronize()
    return {n: getattr(buf, n).cpu().numpy() for n in KEYS}


def test_static_scratch_size():
    assert L.moe_static_scratch_bytes() == 8 << 20


def test_static_equals_workspace_entry_point(ctx, decode_layer):
    """Two calls in a row, 16 tokens (the two-call path inside: h rows of
    128 pairs in the scratch) then 1 token (routing inside the gate/up
    kernel): each bit-identical to moe_decode_layer, and within the decode
    tolerance of the oracle."""
    rl, wl = decode_layer, decode_layer.wl
    wr = dev(gi.router_weight(wl, 0))
    for T in (16, 1):
        note(f"static decode layer T={T}")
        x = gi.activations(wl, T)
        xd = dev(x)
        want = _read(_run(ctx, rl, T, xd, wr, "layer"))
        got_buf = _run(ctx, rl, T, xd, wr, "static")
        got = _read(got_buf)
        moe.moe_ctx_check(ctx)
        for n in KEYS:
            np.testing.assert_array_equal(got[n], want[n], err_msg=f"T={T} {n}")
        ref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, router_w=gi.router_weight(wl, 0))
        check_routed_layer(got["ids"], got["w"], got["logits"], got["y"], got["out"], ref, 1e-3, T,
                           lambda lo: oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, logits=lo))


def test_static_in_graph_replays(ctx, decode_layer):
    """Captured in a HIP graph (the caller that cannot allocate) and replayed
    three times with eager calls between the replays: every replay equals
    moe_decode_layer."""
    rl, wl = decode_layer, decode_layer.wl
    wr = dev(gi.router_weight(wl, 0))
    xs = [dev(gi.activations(wl, T, 3)) for T in (4, 1)]
    wants = [_read(_run(ctx, rl, x.shape[0], x, wr, "layer")) for x in xs]
    bufs = [_poisoned(wl, x.shape[0]) for x in xs]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for b, x in zip(bufs, xs):
            _run(ctx, rl, x.shape[0], x, wr, "static", buf=b)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for b, x in zip(bufs, xs):
            _run(ctx, rl, x.shape[0], x, wr, "static", buf=b)
    for rep in range(3):
        for b in bufs:
            for name in ("y", "out"):
                getattr(b, name).fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        for b, want in zip(bufs, wants):
            got = _read(b)
            for n in KEYS:
                np.testing.assert_array_equal(got[n], want[n], err_msg=f"replay {rep} {n}")
        _run(ctx, rl, 16, dev(gi.activations(wl, 16)), wr, "static")  # an eager call between replays
        torch.cuda.synchronize()
    moe.moe_ctx_check(ctx)


def test_static_refuses_oversized_batch(ctx, decode_layer):
    """A batch whose h rows exceed the static array is refused on the host
    (MOE_ERR_WORKSPACE), before any launch, and leaves the outputs as they
    were."""
    rl, wl = decode_layer, decode_layer.wl
    T = 400  # 400 x 8 pairs x 768 x 4 B = 9.8 MB > 8 MiB
    buf = _poisoned(wl, T)
    with pytest.raises(moe.MoeError) as ei:
        _run(ctx, rl, T, dev(gi.activations(wl, T)), dev(gi.router_weight(wl, 0)), "static", buf=buf)
    assert ei.value.name == "MOE_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert torch.isnan(buf.out).all()
