"""Prefill layer streaming on the GPU: layers whose experts stream from a
pinned host pool through two device buffers (prefill_stream_*) give the
oracle's outputs, bit for bit the resident path's, in any call order, with
the copies as HSA asynchronous copies (the default) and as hipMemcpyAsync
on the copy stream (MOE_STREAM_HIP_COPY=1 at create time)."""
import numpy as np
import pytest
import torch

import expert_offload_amd as moe
from expert_offload_amd import _lib as L
from expert_offload_amd import layer
from gen import inputs as gi
import oracle

from gpu_util import DEV, ResidentLayer, bf16_tensor, dev, max_rel_err, note

pytestmark = pytest.mark.gpu

PREFILL_TOL = 2e-2
SMALL = gi.Workload(7, "stream_small_q4_0", H=512, E=16, k=4, I=256, qtype="q4_0", batches=(300,), layers=3,
                    x_dtype="bf16", router="logits")


@pytest.fixture(scope="module")
def ctx():
    c = moe.Ctx(0)
    yield c
    c.close()


def host_pool(wl):
    """Pinned [L][E] pool of packed experts and the blocks per (layer, expert)."""
    sb = moe.moe_slot_bytes(L.QTYPE[wl.qtype], wl.H, wl.I)
    pool = torch.empty(wl.layers * wl.E * sb, dtype=torch.uint8, pin_memory=True)
    view = pool.numpy()
    blocks = {}

    def put(l, e, b):
        blocks[(l, e)] = b
        view[(l * wl.E + e) * sb:(l * wl.E + e + 1) * sb] = layer.pack_expert(wl.qtype, wl.H, wl.I, *b)

    gi.generate_blocks_parallel(wl, [(l, e) for l in range(wl.layers) for e in range(wl.E)], put)
    return pool, blocks


def resident_out(ctx, wl, blocks, l, T, xd, logits):
    rl = ResidentLayer(wl, layer_idx=l, blocks={e: blocks[(l, e)] for e in range(wl.E)})
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV, mode=L.MODE_PREFILL,
                             x_dtype=L.DTYPE_BF16)
    out = layer.forward(ctx, buf, rl.pool.base(), rl.pool.slot_bytes, rl.pool.n_slots, rl.slot_table, xd,
                        logits_in=dev(logits))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("copies", ["hsa", "hip"])
def test_streamed_layers_match_oracle(ctx, copies, monkeypatch):
    """Three layers called in order twice, then out of order: every call of a
    layer gives the same bytes, equal to the resident path and within the
    prefill tolerance of the oracle; prefetches and demand loads are those
    the dual-buffer schedule implies.  The layers' experts differ, so a
    buffer refilled while stale bytes of its previous layer were still
    visible to the kernels would show here."""
    wl = SMALL
    T = wl.batches[0]
    pool, blocks = host_pool(wl)
    xbits = gi.activations(wl, T)
    x32, xd = gi.bf16_bits_to_f32(xbits), bf16_tensor(xbits)
    logits = [gi.given_logits(wl, T, l) for l in range(wl.layers)]
    logits_d = [dev(g) for g in logits]
    if copies == "hip":
        monkeypatch.setenv("MOE_STREAM_HIP_COPY", "1")
    sp = layer.StreamedPrefill(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, T, pool)
    monkeypatch.delenv("MOE_STREAM_HIP_COPY", raising=False)
    order = [0, 1, 2, 0, 1, 2, 2, 0, 1]
    outs, ids = [], []
    for l in order:
        o = torch.full((T, wl.H), float("nan"), dtype=torch.float32, device=DEV)
        sp.layer(l, xd, logits_d[l], out=o)
        outs.append(o)
        ids.append(sp.buf.ids[:T].clone())
    torch.cuda.synchronize()
    moe.moe_ctx_check(ctx)
    assert sp.stats() == (9, 3)
    first = {}
    for l, o, i in zip(order, outs, ids):
        o = o.cpu().numpy()
        if l in first:
            np.testing.assert_array_equal(o, first[l][0])
            np.testing.assert_array_equal(i.cpu().numpy(), first[l][1])
        else:
            first[l] = (o, i.cpu().numpy())
    for l in range(wl.layers):
        o, i = first[l]
        np.testing.assert_array_equal(o, resident_out(ctx, wl, blocks, l, T, xd, logits[l]))
        ref = oracle.moe_layer(x32, wl.qtype, lambda e: blocks[(l, e)], wl.k, logits=logits[l])
        np.testing.assert_array_equal(i, ref["ids"])
        err = max_rel_err(o, ref["out"])
        note(f"   streamed layer {l}: out max rel err {err:.2e}")
        assert err <= PREFILL_TOL
    sp.close()


def test_streamed_layer_shorter_prompt_and_errors(ctx):
    """A call with fewer tokens than the buffers were made for, T=0, and the
    documented argument errors."""
    wl = SMALL
    T = 37
    pool, blocks = host_pool(wl)
    xbits = gi.activations(wl, T)
    x32, xd = gi.bf16_bits_to_f32(xbits), bf16_tensor(xbits)
    lg = gi.given_logits(wl, T, 1)
    sp = layer.StreamedPrefill(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, 300, pool)
    out = torch.full((T, wl.H), float("nan"), dtype=torch.float32, device=DEV)
    sp.layer(1, xd, dev(lg), out=out)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(x32, wl.qtype, lambda e: blocks[(1, e)], wl.k, logits=lg)
    assert max_rel_err(out.cpu().numpy(), ref["out"]) <= PREFILL_TOL
    with pytest.raises(moe.MoeError) as ei:
        sp.layer(3, xd, dev(lg), out=out)
    assert ei.value.name == "MOE_ERR_INVALID_ARG"
    b = sp.buf
    bad = L.make_ffn_args(None, sp.slot_bytes, wl.E, sp.q, wl.H, 512, T, wl.k, wl.E, None, xd, b.offsets,
                          b.sorted_pairs, b.active, b.y, L.MODE_PREFILL, ws=b.ws, ws_bytes=b.ws.numel(),
                          x_dtype=L.DTYPE_BF16, topk_w=b.w, out=out)
    with pytest.raises(moe.MoeError):  # I differs from the stream's
        moe.prefill_stream_layer(sp.ps, ctx, 0, bad, None, None, dev(lg), None, b.ids, b.pair_pos, None, 0,
                                 sp.copy_stream, None)
    plain = np.zeros(wl.layers * wl.E * sp.slot_bytes, dtype=np.uint8)
    with pytest.raises(moe.MoeError) as ei:
        moe.prefill_stream_create(wl.layers, wl.E, sp.q, wl.H, wl.I, sp.d_bufs, plain.ctypes.data)
    assert ei.value.name == "MOE_ERR_NOT_PINNED"
    sp.close()


def test_streamed_prefill_full_size(ctx):
    """The 4096-token prefill shape over two streamed layers: bit for bit the
    resident path, and 32 sampled tokens of each layer against the oracle."""
    wl = gi.Workload(3, "prefill_q4_0_h2048_e128", H=2048, E=128, k=8, I=768, qtype="q4_0", batches=(4096,),
                     layers=2, x_dtype="bf16", router="logits")
    T = wl.batches[0]
    note("streamed prefill, 2 layers of the 4096-token shape")
    pool, blocks = host_pool(wl)
    xbits = gi.activations(wl, T)
    x32, xd = gi.bf16_bits_to_f32(xbits), bf16_tensor(xbits)
    logits = [gi.given_logits(wl, T, l) for l in range(wl.layers)]
    sp = layer.StreamedPrefill(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, T, pool)
    outs = []
    for l in range(wl.layers):
        o = torch.full((T, wl.H), float("nan"), dtype=torch.float32, device=DEV)
        sp.layer(l, xd, dev(logits[l]), out=o)
        outs.append(o)
    torch.cuda.synchronize()
    moe.moe_ctx_check(ctx)
    assert sp.stats() == (2, 1)
    rng = np.random.default_rng(11)
    for l in range(wl.layers):
        o = outs[l].cpu().numpy()
        np.testing.assert_array_equal(o, resident_out(ctx, wl, blocks, l, T, xd, logits[l]))
        sample = np.sort(rng.choice(T, 32, replace=False))
        ref = oracle.moe_layer(x32[sample], wl.qtype, lambda e: blocks[(l, e)], wl.k, logits=logits[l][sample])
        err = max_rel_err(o[sample], ref["out"])
        note(f"   layer {l}: sampled out max rel err {err:.2e}")
        assert err <= PREFILL_TOL
    sp.close()
