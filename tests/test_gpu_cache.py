"""Expert cache on the GPU: the library's global LRU agrees exactly with the
oracle's simulation, prefetched experts give the oracle's layer outputs,
and the documented errors (unpinned pool, capacity, unmarked layer) fire."""
import numpy as np
import pytest
import torch

import expert_offload_amd as moe
from expert_offload_amd import _lib as L
from expert_offload_amd import layer
from gen import inputs as gi
import oracle

from gpu_util import DEV, dev, max_rel_err, note

pytestmark = pytest.mark.gpu

SMALL = gi.Workload(6, "cache_small_q4_0", H=512, E=16, k=4, I=256, qtype="q4_0", batches=(1,),
                    layers=3, router="trace", cache_fraction=0.6, steps=40, trace_keep_p=0.7,
                    trace_zipf_s=1.0)


@pytest.fixture(scope="module")
def ctx():
    c = moe.Ctx(0)
    yield c
    c.close()


def host_pool(wl):
    sb = moe.moe_slot_bytes(L.QTYPE[wl.qtype], wl.H, wl.I)
    pool = torch.empty(wl.layers * wl.E * sb, dtype=torch.uint8, pin_memory=True)
    view = pool.numpy()
    blocks = {}

    def put(l, e, b):
        blocks[(l, e)] = b
        view[(l * wl.E + e) * sb:(l * wl.E + e + 1) * sb] = layer.pack_expert(wl.qtype, wl.H, wl.I, *b)

    gi.generate_blocks_parallel(wl, [(l, e) for l in range(wl.layers) for e in range(wl.E)], put)
    return pool, blocks


def lookup_order(wl, trace):
    """Per (step, layer) the ids in the order the router emits them (oracle top-k)."""
    order = np.empty_like(trace)
    for s in range(trace.shape[0]):
        lg = gi.cache_trace_logits(wl, trace, s)
        order[s] = oracle.topk_select(lg, wl.k)
    return order


@pytest.mark.parametrize("n_slots", [6, 10, 30])
def test_lru_matches_oracle(ctx, n_slots):
    wl = SMALL
    pool, _ = host_pool(wl)
    trace = lookup_order(wl, gi.cache_trace(wl))
    sb = moe.moe_slot_bytes(L.QTYPE[wl.qtype], wl.H, wl.I)
    d_pool = torch.zeros((n_slots + 2) * sb, dtype=torch.uint8, device=DEV)
    cache = moe.cache_slot_table_create(wl.layers, wl.E, n_slots, L.QTYPE[wl.qtype], wl.H, wl.I, d_pool, pool)
    copy_s = torch.cuda.Stream()
    s = torch.cuda.current_stream()
    hits = np.zeros(trace.shape, dtype=bool)
    for st in range(trace.shape[0]):
        for l in range(wl.layers):
            slots, misses = moe.cache_slot_table_lookup(cache, l, trace[st, l])
            assert len(set(slots.tolist())) == wl.k and (slots >= 0).all() and (slots < n_slots + 2).all()
            hits[st, l] = ~np.isin(trace[st, l], misses)
            for e in misses:
                moe.prefetch_expert(cache, l, int(e), copy_s, s)
            moe.cache_mark_layer_done(cache, l, s)
    torch.cuda.synchronize()
    want, _ = oracle.lru_simulate(trace, n_slots)
    np.testing.assert_array_equal(hits, want)
    h, m = moe.cache_slot_table_stats(cache)
    assert h == int(want.sum()) and m == int((~want).sum())
    # device table: resident keys map to distinct slots whose bytes are the expert's
    table = torch.empty(wl.layers * wl.E, dtype=torch.int32, device=DEV)
    table.copy_(torch.from_dlpack(_table_view(cache, wl)))
    t = table.cpu().numpy()
    res = t[t >= 0]
    assert len(res) == len(set(res.tolist())) <= n_slots
    dp = d_pool.cpu().numpy()
    hp = pool.numpy()
    for key in np.flatnonzero(t >= 0)[:8]:
        np.testing.assert_array_equal(dp[t[key] * sb:(t[key] + 1) * sb], hp[key * sb:(key + 1) * sb])
    cache.close()


def _table_view(cache, wl):
    ptr = moe.cache_slot_table_device(cache)
    n = wl.layers * wl.E

    class _Arr:
        __cuda_array_interface__ = {"shape": (n,), "typestr": "<i4", "data": (ptr, False), "version": 3}
    return torch.as_tensor(_Arr(), device=DEV)


def test_cached_layers_match_oracle(ctx):
    wl = SMALL
    pool, blocks = host_pool(wl)
    trace = gi.cache_trace(wl)
    cl = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, 8, pool)
    worst = 0.0
    for st in range(12):
        x = gi.activations(wl, 1, st)
        lg = gi.cache_trace_logits(wl, trace, st)
        xd = dev(x)
        for l in range(wl.layers):
            out = cl.layer(l, xd, dev(lg[l:l + 1])).cpu().numpy()
            moe.moe_ctx_check(ctx)
            ref = oracle.moe_layer(x, wl.qtype, lambda e: blocks[(l, e)], wl.k, logits=lg[l:l + 1])
            worst = max(worst, max_rel_err(out, ref["out"]))
    note(f"   cached layers worst max rel err {worst:.2e}, misses {sum(cl.misses_per_layer)}")
    assert worst <= 1e-3
    assert sum(cl.misses_per_layer) > 0
    cl.close()


def test_unpinned_pool_refused(ctx):
    wl = SMALL
    sb = moe.moe_slot_bytes(L.QTYPE[wl.qtype], wl.H, wl.I)
    d_pool = torch.zeros(6 * sb, dtype=torch.uint8, device=DEV)
    plain = np.zeros(wl.layers * wl.E * sb, dtype=np.uint8)
    with pytest.raises(moe.MoeError) as ei:
        moe.cache_slot_table_create(wl.layers, wl.E, 4, L.QTYPE[wl.qtype], wl.H, wl.I, d_pool, plain.ctypes.data)
    assert ei.value.name == "MOE_ERR_NOT_PINNED"


def test_capacity_and_unmarked_layer_errors(ctx):
    wl = SMALL
    sb = moe.moe_slot_bytes(L.QTYPE[wl.qtype], wl.H, wl.I)
    pool = torch.zeros(wl.layers * wl.E * sb, dtype=torch.uint8, pin_memory=True)
    d_pool = torch.zeros(5 * sb, dtype=torch.uint8, device=DEV)
    cache = moe.cache_slot_table_create(wl.layers, wl.E, 3, L.QTYPE[wl.qtype], wl.H, wl.I, d_pool, pool)
    with pytest.raises(moe.MoeError) as ei:
        moe.cache_slot_table_lookup(cache, 0, [1, 2, 3, 4])
    assert ei.value.name == "MOE_ERR_CAPACITY"
    assert moe.cache_slot_table_stats(cache) == (0, 0)  # unchanged
    moe.cache_slot_table_lookup(cache, 0, [1, 2])
    with pytest.raises(moe.MoeError) as ei:
        moe.cache_slot_table_lookup(cache, 1, [1, 2])
    assert ei.value.name == "MOE_ERR_INVALID_ARG"
    moe.cache_mark_layer_done(cache, 0, None)
    slots, misses = moe.cache_slot_table_lookup(cache, 1, [1, 2])
    assert misses.tolist() == [1, 2]
    with pytest.raises(moe.MoeError) as ei:
        moe.prefetch_expert(cache, 1, 5, None, None)  # never looked up
    assert ei.value.name == "MOE_ERR_NOT_RESIDENT"
    moe.cache_mark_layer_done(cache, 1, None)
    torch.cuda.synchronize()
    cache.close()


def test_cached_layer_full_size_sampled(ctx):
    """One layer at the expert-cache workload's full shape (hidden 4096, 256
    experts, top-8, intermediate 2048, Q4_0) through a 12-slot cache, so
    later steps evict; only the experts the trace touches get content."""
    import dataclasses
    wl = dataclasses.replace(gi.workload("cache_q4_0_h4096_e256"), layers=1, steps=6)
    sb = moe.moe_slot_bytes(L.QTYPE[wl.qtype], wl.H, wl.I)
    trace = gi.cache_trace(wl)
    touched = sorted(set(trace.reshape(-1).tolist()))
    pool = torch.zeros(wl.E * sb, dtype=torch.uint8, pin_memory=True)
    view = pool.numpy()
    blocks = {}

    def put(l, e, b):
        blocks[e] = b
        view[e * sb:(e + 1) * sb] = layer.pack_expert(wl.qtype, wl.H, wl.I, *b)

    gi.generate_blocks_parallel(wl, [(0, e) for e in touched], put)
    cl = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, 1, 12, pool)
    outs = []
    for st in range(wl.steps):
        x = gi.activations(wl, 1, st)
        lg = gi.cache_trace_logits(wl, trace, st)
        outs.append((x, lg, cl.layer(0, dev(x), dev(lg)).cpu().numpy()))
    moe.moe_ctx_check(ctx)
    assert sum(cl.misses_per_layer[1:]) > 0  # later steps missed, so slots were reused
    for st in (0, 3, wl.steps - 1):
        x, lg, out = outs[st]
        ref = oracle.moe_layer(x, wl.qtype, lambda e: blocks[e], wl.k, logits=lg)
        err = max_rel_err(out, ref["out"])
        note(f"   full-size cached step {st}: max rel err {err:.2e}")
        assert err <= 1e-3
    cl.close()


def test_native_layer_equals_stepwise(ctx):
    """cache_decode_layer (one call per layer) gives the outputs and the hit /
    miss sequence of the same calls made one by one from Python."""
    wl = SMALL
    pool, _ = host_pool(wl)
    trace = gi.cache_trace(wl)
    a = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, 8, pool)
    b = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, 8, pool)
    for st in range(12):
        x = dev(gi.activations(wl, 1, st))
        lg = gi.cache_trace_logits(wl, trace, st)
        for l in range(wl.layers):
            oa = a.layer(l, x, dev(lg[l:l + 1]), native=True).cpu().numpy()
            ob = b.layer(l, x, dev(lg[l:l + 1]), native=False).cpu().numpy()
            np.testing.assert_array_equal(oa, ob, err_msg=f"step {st} layer {l}")
    moe.moe_ctx_check(ctx)
    assert a.misses_per_layer == b.misses_per_layer
    assert a.stats() == b.stats()
    a.close()
    b.close()


def _oracle_resident(trace, hits, evicted):
    """Keys resident at the end of an oracle run: misses insert, evictions
    remove; within one (step, layer) the evictions come first (a key looked
    up in a call is not evicted by it)."""
    res = set()
    ev = {}
    for s, l, key in evicted:
        ev.setdefault((s, l), []).append(key)
    for s in range(trace.shape[0]):
        for l in range(trace.shape[1]):
            for key in ev.get((s, l), []):
                res.discard(key)
            for j in range(trace.shape[2]):
                if not hits[s, l, j]:
                    res.add((l, int(trace[s, l, j])))
    return res


def test_resize_matches_oracle(ctx):
    """Shrink in place, grow into a new pool, shrink into a new pool, in the
    middle of a trace: hits, misses and the resident set follow the oracle's
    LRU with the same capacity schedule, and every resident slot holds its
    expert's bytes after the moves."""
    wl = SMALL
    pool, _ = host_pool(wl)
    trace = lookup_order(wl, gi.cache_trace(wl))
    q = L.QTYPE[wl.qtype]
    sb = moe.moe_slot_bytes(q, wl.H, wl.I)
    schedule = {(10, 0): (12, "in_place"), (20, 1): (20, "new"), (30, 2): (6, "new"), (35, 0): (6, "in_place")}
    n_slots = 30
    d_pool = torch.zeros((n_slots + 2) * sb, dtype=torch.uint8, device=DEV)
    cache = moe.cache_slot_table_create(wl.layers, wl.E, n_slots, q, wl.H, wl.I, d_pool, pool)
    copy_s = torch.cuda.Stream()
    s = torch.cuda.current_stream()
    hp = pool.numpy()
    hits = np.zeros(trace.shape, dtype=bool)

    def check_bytes(n):
        t = _table_view(cache, wl).cpu().numpy()
        res = t[t >= 0]
        assert len(res) == len(set(res.tolist())) <= n and (res < n + 2).all()
        dp = d_pool.cpu().numpy()
        for key in np.flatnonzero(t >= 0):
            np.testing.assert_array_equal(dp[t[key] * sb:(t[key] + 1) * sb], hp[key * sb:(key + 1) * sb])
        return {(int(key) // wl.E, int(key) % wl.E) for key in np.flatnonzero(t >= 0)}

    for st in range(trace.shape[0]):
        for l in range(wl.layers):
            if (st, l) in schedule:
                n_slots, how = schedule[(st, l)]
                if how == "new":
                    new_pool = torch.full(((n_slots + 2) * sb,), 0xA5, dtype=torch.uint8, device=DEV)
                    moe.cache_slot_table_resize(cache, n_slots, new_pool, s)
                    d_pool = new_pool
                else:
                    moe.cache_slot_table_resize(cache, n_slots, None, s)
                note(f"   resize at step {st} layer {l} -> {n_slots} slots ({how})")
                check_bytes(n_slots)
            slots, misses = moe.cache_slot_table_lookup(cache, l, trace[st, l])
            assert (slots >= 0).all() and (slots < n_slots + 2).all()
            hits[st, l] = ~np.isin(trace[st, l], misses)
            for e in misses:
                moe.prefetch_expert(cache, l, int(e), copy_s, s)
            moe.cache_mark_layer_done(cache, l, s)
    torch.cuda.synchronize()
    resizes = {k: v[0] for k, v in schedule.items()}
    want, evicted = oracle.lru_simulate(trace, 30, resizes=resizes)
    np.testing.assert_array_equal(hits, want)
    assert moe.cache_slot_table_stats(cache) == (int(want.sum()), int((~want).sum()))
    assert check_bytes(n_slots) == _oracle_resident(trace, want, evicted)
    cache.close()


def test_resize_errors(ctx):
    wl = SMALL
    q = L.QTYPE[wl.qtype]
    sb = moe.moe_slot_bytes(q, wl.H, wl.I)
    pool = torch.zeros(wl.layers * wl.E * sb, dtype=torch.uint8, pin_memory=True)
    d_pool = torch.zeros(8 * sb, dtype=torch.uint8, device=DEV)
    cache = moe.cache_slot_table_create(wl.layers, wl.E, 6, q, wl.H, wl.I, d_pool, pool)
    moe.cache_slot_table_lookup(cache, 0, [1, 2])
    with pytest.raises(moe.MoeError) as ei:  # misses looked up, copies not issued
        moe.cache_slot_table_resize(cache, 4)
    assert ei.value.name == "MOE_ERR_INVALID_ARG"
    for e in (1, 2):
        moe.prefetch_expert(cache, 0, e, torch.cuda.Stream(), torch.cuda.current_stream())
    with pytest.raises(moe.MoeError):  # layer not marked done
        moe.cache_slot_table_resize(cache, 4)
    moe.cache_mark_layer_done(cache, 0)
    with pytest.raises(moe.MoeError):
        moe.cache_slot_table_resize(cache, 0)
    moe.cache_slot_table_resize(cache, 1)  # keeps expert 2, the most recent
    slots, misses = moe.cache_slot_table_lookup(cache, 0, [2])
    assert len(misses) == 0
    moe.cache_mark_layer_done(cache, 0)
    torch.cuda.synchronize()
    cache.close()


def test_cached_layers_resize_outputs(ctx):
    """Layer outputs through the cache stay the oracle's across run-time
    resizes (in place and into a new pool)."""
    wl = SMALL
    pool, blocks = host_pool(wl)
    trace = gi.cache_trace(wl)
    cl = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, 12, pool)
    plan = {4: (5, True), 8: (14, False), 11: (4, False)}
    worst = 0.0
    for st in range(14):
        if st in plan:
            cl.resize(plan[st][0], in_place=plan[st][1])
        x = gi.activations(wl, 1, st)
        lg = gi.cache_trace_logits(wl, trace, st)
        xd = dev(x)
        for l in range(wl.layers):
            out = cl.layer(l, xd, dev(lg[l:l + 1]), native=(st % 2 == 0)).cpu().numpy()
            moe.moe_ctx_check(ctx)
            ref = oracle.moe_layer(x, wl.qtype, lambda e: blocks[(l, e)], wl.k, logits=lg[l:l + 1])
            worst = max(worst, max_rel_err(out, ref["out"]))
    note(f"   cached layers with resizes: worst max rel err {worst:.2e}")
    assert worst <= 1e-3
    cl.close()


def _run_policies(ctx, wl, pool, blocks, n_slots, plan, steps):
    """Native cached layers under a per-step miss policy; returns the
    per-(step, layer) host and copied ids, misses and the worst output
    error against the oracle."""
    raw = gi.cache_trace(wl)
    trace = lookup_order(wl, raw)
    cl = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, n_slots, pool)
    host, copied, computed, worst = {}, {}, {}, 0.0
    for st in range(steps):
        if st in plan:
            cl.set_miss_policy(plan[st], host_threads=4)
        x = gi.activations(wl, 1, st)
        lg = gi.cache_trace_logits(wl, raw, st)
        xd = dev(x)
        for l in range(wl.layers):
            out = cl.layer(l, xd, dev(lg[l:l + 1])).cpu().numpy()
            moe.moe_ctx_check(ctx)
            cp, hs, n_only = cl.last_misses()
            host[(st, l)], copied[(st, l)] = set(hs[:n_only].tolist()), cp.tolist()
            computed[(st, l)] = set(hs.tolist())
            ref = oracle.moe_layer(x, wl.qtype, lambda e: blocks[(l, e)], wl.k, logits=lg[l:l + 1])
            worst = max(worst, max_rel_err(out, ref["out"]))
    misses = np.array(cl.misses_per_layer).reshape(steps, wl.layers)
    stats = cl.miss_stats()
    cl.close()
    return trace[:steps], host, copied, computed, misses, worst, stats


def test_miss_policies_match_oracle(ctx):
    """Copy, host and Q* policies in turn: layer outputs stay within the
    decode tolerance of the oracle, and the cache follows the oracle's LRU
    given the experts the library computed on the host (misses per layer,
    and the copied experts in router order)."""
    wl = SMALL
    pool, blocks = host_pool(wl)
    plan = {0: L.MISS_COPY, 8: L.MISS_HOST, 16: L.MISS_QSTAR, 24: L.MISS_COPY}
    trace, host, copied, computed, misses, worst, stats = _run_policies(ctx, wl, pool, blocks, 8, plan, 30)
    note(f"   policies: worst max rel err {worst:.2e}; copied {stats[0]}, host {stats[1]}, "
         f"rates {stats[2]:.1f} / {stats[3]:.1f} GB/s")
    assert worst <= 1e-3
    assert stats[1] > 0 and stats[0] > 0
    assert all(not host[(s, l)] for s in range(8) for l in range(wl.layers))
    want, _ = oracle.lru_simulate(trace, 8, host=host)
    np.testing.assert_array_equal(misses, (~want).sum(axis=2))
    for (s, l), cp in copied.items():
        order = []
        for j in range(wl.k):
            e = int(trace[s, l, j])
            if not want[s, l, j] and e not in host[(s, l)] and e not in order:
                order.append(e)
        assert cp == order, (s, l)
    for s in range(8, 16):  # the host policy copies nothing
        assert all(not copied[(s, l)] for l in range(wl.layers))


def test_host_policy_full_size_sampled(ctx):
    """The expert-cache workload's shape (hidden 4096, intermediate 2048,
    Q4_0) with every miss on the host for a few steps: outputs within the
    decode tolerance of the oracle."""
    wl = gi.workload("cache_q4_0_h4096_e256")
    wl = gi.Workload(wl.index, wl.name, H=wl.H, E=wl.E, k=wl.k, I=wl.I, qtype=wl.qtype, batches=(1,), layers=1,
                     router="trace", cache_fraction=wl.cache_fraction, steps=4, trace_keep_p=wl.trace_keep_p,
                     trace_zipf_s=wl.trace_zipf_s)
    trace = gi.cache_trace(wl, 4)
    need = sorted({(0, int(e)) for e in trace.reshape(-1)})
    sb = moe.moe_slot_bytes(L.QTYPE[wl.qtype], wl.H, wl.I)
    pool = torch.zeros(wl.E * sb, dtype=torch.uint8, pin_memory=True)
    view = pool.numpy()
    blocks = {}

    def put(l, e, b):
        blocks[(l, e)] = b
        view[e * sb:(e + 1) * sb] = layer.pack_expert(wl.qtype, wl.H, wl.I, *b)

    gi.generate_blocks_parallel(wl, need, put)
    cl = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, 1, 16, pool)
    cl.set_miss_policy(L.MISS_HOST)
    worst = 0.0
    for st in range(4):
        x = gi.activations(wl, 1, st)
        lg = gi.cache_trace_logits(wl, trace, st)
        out = cl.layer(0, dev(x), dev(lg[0:1])).cpu().numpy()
        moe.moe_ctx_check(ctx)
        ref = oracle.moe_layer(x, wl.qtype, lambda e: blocks[(0, e)], wl.k, logits=lg[0:1])
        worst = max(worst, max_rel_err(out, ref["out"]))
    assert cl.miss_stats()[1] == cl.stats()[1] > 0
    note(f"   host policy at full size: worst max rel err {worst:.2e}")
    assert worst <= 1e-3
    cl.close()


def test_host_copy_policy_keeps_the_lru(ctx):
    """Misses computed on the host while their copies run behind: the cache
    follows the plain LRU (every miss inserted), every copied expert was
    also computed on the host, and outputs stay within the decode tolerance
    of the oracle."""
    wl = SMALL
    pool, blocks = host_pool(wl)
    trace, host, copied, computed, misses, worst, stats = _run_policies(ctx, wl, pool, blocks, 8,
                                                                        {0: L.MISS_HOST_COPY}, 30)
    note(f"   host+copy: worst max rel err {worst:.2e}; copied {stats[0]}, host {stats[1]}, "
         f"left out {sum(len(h) for h in host.values())}")
    assert worst <= 1e-3
    want, _ = oracle.lru_simulate(trace, 8, host=host)
    np.testing.assert_array_equal(misses, (~want).sum(axis=2))
    for key, cp in copied.items():
        assert set(cp) <= computed[key] and not (set(cp) & host[key])
    assert stats[1] >= stats[0] > 0


def test_widest_cache_masks_match_oracle(ctx):
    """1024 experts, the most a cache takes: the hit / copied / host masks,
    which travel to the device as bits, cover ids across every word, under
    the copy, host and host-now-copy-behind policies in turn; outputs within
    the decode tolerance of the oracle and misses as its LRU has them."""
    wl = gi.Workload(9, "cache_widest_q4_0", H=256, E=1024, k=8, I=256, qtype="q4_0", batches=(1,),
                     layers=1, router="trace", cache_fraction=0.06, steps=12, trace_keep_p=0.5,
                     trace_zipf_s=1.0)
    pool, blocks = host_pool(wl)
    plan = {0: L.MISS_COPY, 4: L.MISS_HOST, 8: L.MISS_HOST_COPY}
    trace, host, copied, computed, misses, worst, stats = _run_policies(ctx, wl, pool, blocks, 64, plan, 12)
    note(f"   widest cache: worst max rel err {worst:.2e}; copied {stats[0]}, host {stats[1]}")
    assert worst <= 1e-3
    assert stats[0] > 0 and stats[1] > 0
    assert (trace >= 512).any() and (trace < 512).any()
    want, _ = oracle.lru_simulate(trace, 64, host=host)
    np.testing.assert_array_equal(misses, (~want).sum(axis=2))


def test_lru_full_expert_cache_trace(ctx):
    """The expert-cache workload's whole trace (8 layers, 256 experts,
    top-8, 2048 single-token steps, 816 slots = 40% of each layer's
    experts) through cache_decode_layer, the call the benchmark makes per
    layer, with experts of a small size (the LRU's decisions do not depend
    on it): every lookup's hit or miss equals the oracle's LRU, and the
    cache's counts equal the oracle's."""
    import dataclasses
    big = gi.workload("cache_q4_0_h4096_e256")
    wl = dataclasses.replace(big, H=256, I=256)
    trace = gi.cache_trace(big)
    steps = trace.shape[0]
    n_slots = int(big.cache_fraction * big.E) * big.layers
    note(f"full expert-cache trace: {steps} steps x {big.layers} layers, {n_slots} slots")
    sb = moe.moe_slot_bytes(L.QTYPE[wl.qtype], wl.H, wl.I)
    pool = torch.zeros(wl.layers * wl.E * sb, dtype=torch.uint8, pin_memory=True)
    logits = np.stack([gi.cache_trace_logits(big, trace, s) for s in range(steps)])
    order = oracle.topk_select(logits, big.k)  # the router's order of each (step, layer)'s ids
    lg = dev(logits)
    x = torch.zeros((1, wl.H), dtype=torch.float32, device=DEV)
    cl = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, n_slots, pool)
    hits = np.zeros(order.shape, dtype=bool)
    for s in range(steps):
        for l in range(wl.layers):
            cl.layer(l, x, lg[s, l:l + 1])
            copied, on_host, _ = cl.last_misses()
            assert len(on_host) == 0
            hits[s, l] = ~np.isin(order[s, l], copied)
        if (s + 1) % 512 == 0:
            note(f"   step {s + 1}")
    torch.cuda.synchronize()
    moe.moe_ctx_check(ctx)
    want, _ = oracle.lru_simulate(order, n_slots)
    np.testing.assert_array_equal(hits, want)
    h, m = cl.stats()
    assert h == int(want.sum()) and m == int((~want).sum())
    note(f"   hit rate {h / (h + m):.4f} ({m} misses), equal to the oracle's on every lookup")
    cl.close()
