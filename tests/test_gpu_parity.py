"""GPU parity of libmoe against the CPU oracle: exact dequantisation, exact
top-k ids and grouping, and layer outputs within tolerance (max relative
error <= 1e-3 for fp32-accumulated decode)."""
import numpy as np
import pytest
import torch

import expert_offload_amd as moe
from expert_offload_amd import _lib as L
from expert_offload_amd import layer
from gen import inputs as gi
import oracle

from gpu_util import DEV, ResidentLayer, check_routed_layer, dev, max_rel_err, note

pytestmark = pytest.mark.gpu

DECODE_TOL = 1e-3
WEIGHT_TOL = 1e-5
NEAR_TIE = 1e-5  # oracle logit gap below which fp32 rounding may reorder experts


@pytest.fixture(scope="module")
def ctx():
    c = moe.Ctx(0)
    yield c
    c.close()


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("qt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("rows,cols", [(3, 256), (17, 768), (64, 2048)])
def test_dequantize_exact(ctx, qt, rows, cols):
    note(f"dequant {qt} {rows}x{cols}")
    rng = np.random.default_rng(rows * cols)
    quant = gi.quantize_q8_0 if qt == "q8_0" else gi.quantize_q4_0
    w = (rng.standard_normal((rows, cols)) * rng.choice([1e-3, 0.02, 3.0, 500.0], (rows, 1)))
    blocks = quant(w.astype(np.float32))
    blocks[0, 0, 0:2] = [0, 0]              # d = 0
    blocks[-1, -1, 0:2] = [0x01, 0x00]      # subnormal d
    packed = np.empty(blocks.size, dtype=np.uint8)
    moe.moe_pack_matrix(L.QTYPE[qt], rows, cols, blocks, packed)
    pd = dev(packed)
    out32 = torch.full((rows, cols), float("nan"), dtype=torch.float32, device=DEV)
    out16 = torch.zeros((rows, cols), dtype=torch.bfloat16, device=DEV)
    moe.moe_dequantize(ctx, L.QTYPE[qt], pd, rows, cols, out32)
    moe.moe_dequantize(ctx, L.QTYPE[qt], pd, rows, cols, out16)
    torch.cuda.synchronize()
    ref = oracle.dequant(qt, blocks)
    ref32 = ref.astype(np.float32)
    assert np.array_equal(ref32.astype(np.float64), ref)  # d*q is exact in fp32
    got32 = out32.cpu().numpy()
    np.testing.assert_array_equal(got32.view(np.uint32), ref32.view(np.uint32))
    got16 = out16.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got16, gi.f32_to_bf16_bits(ref32))


# -------------------------------------------------------------------- route
def _route_given(ctx, logits, k, bias=None):
    T, E = logits.shape
    ids = torch.full((T, k), -5, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    lo = torch.empty((T, E), dtype=torch.float32, device=DEV)
    moe.moe_route(ctx, None, None, None if bias is None else dev(bias), dev(logits), T, 0, E, k,
                  lo, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), lo.cpu().numpy()


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (7, 128, 8), (33, 512, 10), (5, 1024, 64),
                                   (4096, 128, 8), (3, 64, 64), (2, 1, 1)])
def test_topk_exact_given_logits(ctx, T, E, k):
    note(f"topk given logits T={T} E={E} k={k}")
    rng = np.random.default_rng(T * 1000 + E)
    l = rng.standard_normal((T, E)).astype(np.float32)
    # planted exact ties, including ties straddling the k-th place
    l[0, : min(E, 5)] = 0.75
    if T > 1:
        l[1] = np.round(l[1] * 2) / 2
    ids, w, lo = _route_given(ctx, l, k)
    ref_ids = oracle.topk_select(l, k)
    np.testing.assert_array_equal(ids, ref_ids)
    np.testing.assert_array_equal(lo, l)
    ref_w = oracle.renormalize(oracle.softmax(l.astype(np.float64)), ref_ids)
    assert np.abs(w - ref_w).max() <= WEIGHT_TOL * np.abs(ref_w).max()


@pytest.mark.parametrize("E,k", [(512, 10), (256, 8), (1024, 64), (130, 3)])
def test_topk_many_equal_candidates(ctx, E, k):
    """More logits tied at the top than the threshold selection's candidate
    scratch holds (its fallback, k rounds of arg-max, takes over), next to
    rows that fit: lowest ids first among equals, weights uniform."""
    T = 4
    rng = np.random.default_rng(E + k)
    l = rng.standard_normal((T, E)).astype(np.float32)
    l[0] = 1.0                    # every logit equal
    l[1, : E - 1] = 2.5           # all but the last equal and largest
    l[2, rng.permutation(E)[:200 % E]] = 9.0  # a block of equal maxima at random ids
    ids, w, _ = _route_given(ctx, l, k)
    np.testing.assert_array_equal(ids, oracle.topk_select(l, k))
    assert ids[0].tolist() == list(range(k)) and ids[1].tolist() == list(range(k))
    np.testing.assert_allclose(w[0], np.full(k, 1.0 / k), rtol=1e-6)


def test_topk_bias_and_nan(ctx):
    E, k = 16, 4
    l = np.zeros((2, E), dtype=np.float32)
    l[0, 3] = np.nan
    bias = -np.log(np.arange(E) + 1.0).astype(np.float32)
    ids, w, lo = _route_given(ctx, l, k, bias=bias)
    # NaN is never chosen over a finite logit; with the bias, lower ids win
    assert ids[0].tolist() == [0, 1, 2, 4]
    assert ids[1].tolist() == [0, 1, 2, 3]
    np.testing.assert_array_equal(lo[1], bias)


@pytest.mark.parametrize("name,T", [("tiny_q8_0", 4), ("decode_q8_0_h2048_e128", 16),
                                    ("wide_q4_0_h2048_e512", 64), ("tiny_q8_0", 1), ("tiny_q8_0", 3),
                                    ("decode_q8_0_h2048_e128", 13), ("decode_q8_0_h2048_e128", 100),
                                    ("wide_q4_0_h2048_e512", 71)])
def test_router_computed(ctx, name, T):
    note(f"router computed {name} T={T}")
    wl = gi.workload(name)
    x = gi.activations(wl, T)
    wr = gi.router_weight(wl)
    b = gi.router_bias(wl)
    ids = torch.empty((T, wl.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, wl.k), dtype=torch.float32, device=DEV)
    lo = torch.empty((T, wl.E), dtype=torch.float32, device=DEV)
    moe.moe_route(ctx, dev(x), dev(wr), None if b is None else dev(b), None, T, wl.H, wl.E, wl.k,
                  lo, ids, w)
    torch.cuda.synchronize()
    ref_l = oracle.router_logits(x, wr, b)
    got_l = lo.cpu().numpy()
    assert np.abs(got_l - ref_l).max() <= 1e-5 * max(1.0, np.abs(ref_l).max())
    got_ids, got_w = ids.cpu().numpy(), w.cpu().numpy()
    # the exact contract, every token: the oracle's selection and weights on the GPU's own logits
    np.testing.assert_array_equal(got_ids, oracle.topk_select(got_l, wl.k))
    own_w = oracle.renormalize(oracle.softmax(got_l.astype(np.float64)), got_ids)
    assert np.abs(got_w - own_w).max() <= WEIGHT_TOL
    # end to end against the oracle's own logits, near ties counted and reported
    ref_ids, ref_w = oracle.route(ref_l, wl.k)
    ok = oracle.topk_gap(ref_l, wl.k) >= NEAR_TIE
    note(f"   near-tie tokens: {int((~ok).sum())} of {T}")
    np.testing.assert_array_equal(got_ids[ok], ref_ids[ok])
    assert (~ok).sum() <= max(1, T // 100), f"{(~ok).sum()} near-tie tokens"
    assert np.abs(got_w[ok] - ref_w[ok]).max() <= WEIGHT_TOL


def test_router_logits_batch_invariant(ctx):
    """The router kernel takes several tokens per pass (a partial last pass
    repeats a token); each token's logits are bit-identical to those of the
    token routed alone, for batch sizes across the pass widths and past the
    64-token chunk."""
    wl = gi.workload("decode_q8_0_h2048_e128")
    x = gi.activations(wl, 77)
    wr = dev(gi.router_weight(wl))

    def logits(rows):
        T = rows.shape[0]
        lo = torch.empty((T, wl.E), dtype=torch.float32, device=DEV)
        ids = torch.empty((T, wl.k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, wl.k), dtype=torch.float32, device=DEV)
        moe.moe_route(ctx, dev(rows), wr, None, None, T, wl.H, wl.E, wl.k, lo, ids, w)
        torch.cuda.synchronize()
        return lo.cpu().numpy()

    alone = np.stack([logits(x[t:t + 1])[0] for t in range(x.shape[0])])
    for T in (2, 3, 7, 8, 9, 15, 64, 65, 77):
        np.testing.assert_array_equal(logits(x[:T]), alone[:T])


def test_router_logits_experts_per_workgroup(ctx):
    """Past 16 tokens a router workgroup takes four experts; with 10 experts
    the last workgroup holds two past the end (loaded from the last expert's
    row, never written).  Logits against the oracle, and each token's logits
    bit-identical to the token routed alone."""
    wl = gi.Workload(61, "router_h256_e10", H=256, E=10, k=2, I=256, qtype="q8_0", batches=(40,))
    x = gi.activations(wl, 40)
    wr = gi.router_weight(wl)

    def logits(rows):
        T = rows.shape[0]
        lo = torch.full((T, wl.E), float("nan"), dtype=torch.float32, device=DEV)
        ids = torch.empty((T, wl.k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, wl.k), dtype=torch.float32, device=DEV)
        moe.moe_route(ctx, dev(rows), dev(wr), None, None, T, wl.H, wl.E, wl.k, lo, ids, w)
        torch.cuda.synchronize()
        return lo.cpu().numpy()

    got = logits(x)
    ref = oracle.router_logits(x, wr, None)
    assert np.abs(got - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())
    alone = np.stack([logits(x[t:t + 1])[0] for t in range(x.shape[0])])
    for T in (17, 33, 40):
        np.testing.assert_array_equal(logits(x[:T]), alone[:T])


# ------------------------------------------------------------------ permute
@pytest.mark.parametrize("with_ws", [False, True])
@pytest.mark.parametrize("T,k,E", [(0, 2, 8), (1, 1, 1), (4, 2, 8), (16, 8, 128), (64, 10, 512),
                                   (100, 7, 1024), (4096, 8, 128), (513, 3, 5), (600, 7, 1024),
                                   (4113, 8, 128), (2049, 2, 2)])
def test_permute_exact(ctx, T, k, E, with_ws):
    """Exact grouping against the oracle; with the workspace, batches above
    4096 pairs take the chunked multi-workgroup path (last chunk ragged)."""
    note(f"permute T={T} k={k} E={E} ws={with_ws}")
    rng = np.random.default_rng(T + 7 * k + E)
    if T == 0:
        ids = np.zeros((0, k), dtype=np.int32)
    elif E >= k:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32).reshape(T, k)
    else:
        ids = rng.integers(0, E, (T, k)).astype(np.int32)
    if T > 3:
        ids[: T // 2, 0] = 0  # a hot expert (repeats within a token are allowed)
    P = max(T * k, 1)
    off = torch.full((E + 1,), -9, dtype=torch.int32, device=DEV)
    sp = torch.full((P,), -9, dtype=torch.int32, device=DEV)
    pos = torch.full((P,), -9, dtype=torch.int32, device=DEV)
    act = torch.full((E + 1,), -9, dtype=torch.int32, device=DEV)
    nws = moe.moe_permute_workspace_size(T, k, E)
    assert (nws > 0) == (T * k > 4096)
    ws = torch.full((max(nws, 4) // 4,), -3, dtype=torch.int32, device=DEV) if with_ws else None
    moe.moe_permute(ctx, dev(ids) if T else sp, T, k, E, off, sp, pos, act, ws, nws if with_ws else 0)
    torch.cuda.synchronize()
    moe.moe_ctx_check(ctx)
    r_off, r_sp, r_pos, r_act = oracle.permute(ids, E)
    np.testing.assert_array_equal(off.cpu().numpy(), r_off)
    if T:
        np.testing.assert_array_equal(sp.cpu().numpy(), r_sp)
        np.testing.assert_array_equal(pos.cpu().numpy(), r_pos)
    a = act.cpu().numpy()
    assert a[0] == len(r_act)
    np.testing.assert_array_equal(a[1:1 + a[0]], r_act)


# ------------------------------------------------------------- whole layers
def _run_layer(ctx, rl, T, x, wr=None, b=None, logits=None, mode=L.MODE_DECODE, x_dtype=L.DTYPE_F32,
               xd=None, fused=False, repeat=1):
    wl = rl.wl
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV, mode=mode,
                             x_dtype=x_dtype)
    outs = []
    for _ in range(repeat):
        buf.y.fill_(float("nan"))
        buf.out.fill_(float("nan"))
        out = layer.forward(ctx, buf, rl.pool.base(), rl.pool.slot_bytes, rl.pool.n_slots, rl.slot_table,
                            dev(x) if xd is None else xd,
                            router_w=None if wr is None else dev(wr), bias=None if b is None else dev(b),
                            logits_in=None if logits is None else dev(logits), fused=fused)
        torch.cuda.synchronize()
        moe.moe_ctx_check(ctx)
        outs.append(out.cpu().numpy())
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])  # counters were reset between calls
    return buf, outs[0]


def _check_layer(buf, got_out, ref, tol, T, reref=None):
    check_routed_layer(buf.ids.cpu().numpy(), buf.w.cpu().numpy(), buf.logits.cpu().numpy(), buf.y.cpu().numpy(),
                       got_out, ref, tol, T, reref)


def test_tiny_layer(ctx):
    wl = gi.workload("tiny_q8_0")
    T = wl.batches[0]
    rl = ResidentLayer(wl)
    x, wr = gi.activations(wl, T), gi.router_weight(wl)
    buf, out = _run_layer(ctx, rl, T, x, wr)
    ref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, router_w=wr)
    _check_layer(buf, out, ref, DECODE_TOL, T, lambda lo: oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, logits=lo))


@pytest.fixture(scope="module")
def decode_layer():
    return ResidentLayer(gi.workload("decode_q8_0_h2048_e128"), layer_idx=0)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("T", [1, 4, 16, 17, 100])
def test_decode_q8_0_layer(ctx, decode_layer, T, fused):
    """Decode layers at the benchmark's batch sizes, and past 16 tokens,
    where an expert's pairs are split into runs of at most 8 and the top-k
    runs in its own kernel ahead of the grouping."""
    note(f"decode q8_0 layer T={T} fused={fused}")
    wl = decode_layer.wl
    x, wr = gi.activations(wl, T), gi.router_weight(wl, 0)
    buf, out = _run_layer(ctx, decode_layer, T, x, wr, fused=fused, repeat=2)
    ref = oracle.moe_layer(x, wl.qtype, decode_layer.get_blocks, wl.k, router_w=wr)
    _check_layer(buf, out, ref, DECODE_TOL, T,
                 lambda lo: oracle.moe_layer(x, wl.qtype, decode_layer.get_blocks, wl.k, logits=lo))


def test_tiny_layer_fused(ctx):
    wl = gi.workload("tiny_q8_0")
    T = wl.batches[0]
    rl = ResidentLayer(wl)
    x, wr = gi.activations(wl, T), gi.router_weight(wl)
    buf, out = _run_layer(ctx, rl, T, x, wr, fused=True, repeat=3)
    ref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, router_w=wr)
    _check_layer(buf, out, ref, DECODE_TOL, T, lambda lo: oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, logits=lo))


@pytest.fixture(scope="module")
def wide_layer():
    return ResidentLayer(gi.workload("wide_q4_0_h2048_e512"), layer_idx=0)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("T", [1, 64])
def test_wide_q4_0_layer_zipf(ctx, wide_layer, T, fused):
    note(f"wide q4_0 layer T={T} fused={fused}")
    wl = wide_layer.wl
    x, wr, b = gi.activations(wl, T), gi.router_weight(wl, 0), gi.router_bias(wl)
    buf, out = _run_layer(ctx, wide_layer, T, x, wr, b, fused=fused, repeat=2)
    ref = oracle.moe_layer(x, wl.qtype, wide_layer.get_blocks, wl.k, router_w=wr, bias=b)
    _check_layer(buf, out, ref, DECODE_TOL, T,
                 lambda lo: oracle.moe_layer(x, wl.qtype, wide_layer.get_blocks, wl.k, logits=lo))
    counts = np.diff(buf.offsets.cpu().numpy())
    note(f"   active experts {int((counts > 0).sum())}, max tokens per expert {int(counts.max())}")


def test_cache_shaped_q4_0_layer(ctx):
    """H=4096, I=2048, 256 experts, top-8 (one layer, all resident)."""
    wl = gi.workload("cache_q4_0_h4096_e256")
    T = 1
    trace = gi.cache_trace(wl, steps=3)
    ids_needed = sorted(set(int(e) for e in trace[:, 0].ravel()))
    rl = ResidentLayer(wl, layer_idx=0, experts=ids_needed)
    for step in range(3):
        logits = gi.cache_trace_logits(wl, trace, step)[0:1]
        x = gi.activations(wl, T, step)
        for fused in (False, True):
            buf, out = _run_layer(ctx, rl, T, x, logits=logits, fused=fused)
            ref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, logits=logits)
            assert sorted(buf.ids.cpu().numpy()[0].tolist()) == sorted(trace[step, 0].tolist())
            _check_layer(buf, out, ref, DECODE_TOL, T)


@pytest.mark.parametrize("T,E,k,H,given", [(1, 128, 8, 2048, False), (16, 128, 8, 2048, False),
                                           (64, 512, 10, 2048, False), (4, 8, 2, 256, False),
                                           (3, 1024, 64, 256, False), (7, 256, 8, 4096, True),
                                           (500, 128, 8, 2048, True)])
def test_route_permute_fused_equals_separate(ctx, T, E, k, H, given):
    note(f"route_permute T={T} E={E} k={k} given={given}")
    rng = np.random.default_rng(T + E + k)
    x = dev(rng.standard_normal((T, H)).astype(np.float32))
    wr = dev((rng.standard_normal((E, H)) * 0.02).astype(np.float32))
    lg = dev(rng.standard_normal((T, E)).astype(np.float32)) if given else None
    bias = dev(rng.standard_normal(E).astype(np.float32) * 0.1)

    def bufs():
        return dict(lo=torch.full((T, E), np.nan, device=DEV), ids=torch.full((T, k), -7, dtype=torch.int32, device=DEV),
                    w=torch.full((T, k), np.nan, device=DEV), off=torch.full((E + 1,), -7, dtype=torch.int32, device=DEV),
                    sp=torch.full((T * k,), -7, dtype=torch.int32, device=DEV),
                    pos=torch.full((T * k,), -7, dtype=torch.int32, device=DEV),
                    act=torch.full((E + 1,), -7, dtype=torch.int32, device=DEV))
    a, f = bufs(), bufs()
    moe.moe_route(ctx, x, wr, bias, lg, T, H, E, k, a["lo"], a["ids"], a["w"])
    moe.moe_permute(ctx, a["ids"], T, k, E, a["off"], a["sp"], a["pos"], a["act"])
    assert moe.moe_route_permute_workspace_size(T, k, E) == 0
    for _ in range(2):
        moe.moe_route_permute(ctx, x, wr, bias, lg, T, H, E, k, f["lo"], f["ids"], f["w"], f["off"], f["sp"],
                              f["pos"], f["act"], None, 0)
    torch.cuda.synchronize()
    moe.moe_ctx_check(ctx)
    for key in a:
        np.testing.assert_array_equal(a[key].cpu().numpy(), f[key].cpu().numpy(), err_msg=key)


def test_not_resident_expert_gives_nan_and_error(ctx):
    wl = gi.workload("tiny_q8_0")
    T = wl.batches[0]
    rl = ResidentLayer(wl)
    x, wr = gi.activations(wl, T), gi.router_weight(wl)
    ref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, router_w=wr)
    victim = int(ref["ids"][0, 0])
    table = rl.perm.copy()
    table[victim] = -1
    rl.slot_table = dev(table)
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV)
    out = layer.forward(ctx, buf, rl.pool.base(), rl.pool.slot_bytes, rl.pool.n_slots, rl.slot_table, dev(x),
                        router_w=dev(wr)).cpu().numpy()
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_ctx_check(ctx)
    assert ei.value.name == "MOE_ERR_NOT_RESIDENT" and f"expert {victim}" in str(ei.value)
    moe.moe_ctx_check(ctx)  # the word was cleared
    uses = (ref["ids"] == victim).any(axis=1)
    assert np.isnan(out[uses]).all(axis=1).all()
    assert np.isfinite(out[~uses]).all()


# ---------------------------------------------------------------- prefill
PREFILL_TOL = 2e-2


@pytest.fixture(scope="module")
def prefill_layer():
    return ResidentLayer(gi.workload("prefill_q4_0_h2048_e128"), layer_idx=0)


def _prefill_inputs(wl, T):
    logits = gi.given_logits(wl, T)
    xbits = gi.activations(wl, T)
    return logits, xbits, gi.bf16_bits_to_f32(xbits)


@pytest.mark.parametrize("T", [1, 37, 300, 1000])
def test_prefill_layer(ctx, prefill_layer, T):
    """Grouped-GEMM path (bf16 MFMA) against the oracle, ragged expert tiles."""
    note(f"prefill q4_0 layer T={T}")
    wl = prefill_layer.wl
    logits, xbits, x32 = _prefill_inputs(wl, T)
    from gpu_util import bf16_tensor
    buf, out = _run_layer(ctx, prefill_layer, T, x32, logits=logits, mode=L.MODE_PREFILL,
                          x_dtype=L.DTYPE_BF16, xd=bf16_tensor(xbits), repeat=2)
    ref = oracle.moe_layer(x32, wl.qtype, prefill_layer.get_blocks, wl.k, logits=logits)
    np.testing.assert_array_equal(buf.ids.cpu().numpy(), ref["ids"])
    _check_layer(buf, out, ref, PREFILL_TOL, T)


@pytest.mark.parametrize("T", [2048, 4096])
def test_prefill_full_compare(ctx, prefill_layer, T):
    """The launch the prefill bench times, compared element by element on
    every token.  4096 tokens (about 256 pairs per expert: full 256-row tiles
    plus split tails of at most 64 rows) and 2048 tokens (about 128 pairs per
    expert: partial tiles of 65-255 rows taken whole)."""
    wl = prefill_layer.wl
    note(f"prefill full compare T={T}")
    logits, xbits, x32 = _prefill_inputs(wl, T)
    from gpu_util import bf16_tensor
    buf, out = _run_layer(ctx, prefill_layer, T, x32, logits=logits, mode=L.MODE_PREFILL,
                          x_dtype=L.DTYPE_BF16, xd=bf16_tensor(xbits))
    counts = np.diff(buf.offsets.cpu().numpy())
    note(f"   pairs per expert: min {counts.min()} max {counts.max()}; "
         f"{int(((counts % 256) > 64).sum())} experts end in a tile of 65-255 rows")
    ref = oracle.moe_layer(x32, wl.qtype, prefill_layer.get_blocks, wl.k, logits=logits)
    np.testing.assert_array_equal(buf.ids.cpu().numpy(), ref["ids"])
    _check_layer(buf, out, ref, PREFILL_TOL, T)


def test_prefill_layer_graph_replays(ctx, prefill_layer):
    """The prefill layer (routing on given logits, permutation, both grouped
    GEMMs, combine) captured as one HIP graph, as the bench replays it: every
    replay, with the outputs poisoned before it and an eager forward after
    it, equals the eager forward bit for bit, and the eager forward is within
    the prefill tolerance of the oracle.  1000 tokens: partial tiles and
    tails."""
    wl, T = prefill_layer.wl, 1000
    note(f"prefill graph replays T={T}")
    logits, xbits, x32 = _prefill_inputs(wl, T)
    from gpu_util import bf16_tensor
    xd, ld = bf16_tensor(xbits), dev(logits)
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV, mode=L.MODE_PREFILL,
                             x_dtype=L.DTYPE_BF16)

    def run():
        layer.forward(ctx, buf, prefill_layer.pool.base(), prefill_layer.pool.slot_bytes, prefill_layer.pool.n_slots,
                      prefill_layer.slot_table, xd, logits_in=ld)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    s.synchronize()
    moe.moe_ctx_check(ctx)
    eager = {n: getattr(buf, n).clone() for n in ("ids", "w", "offsets", "sorted_pairs", "y", "out")}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    for rep in range(3):
        for n in ("w", "y", "out"):
            getattr(buf, n).fill_(float("nan"))
        buf.ids.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        moe.moe_ctx_check(ctx)
        for n, want in eager.items():
            assert torch.equal(getattr(buf, n), want), f"replay {rep}: {n} differs from the eager forward"
        run()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(buf.out, eager["out"])
    ref = oracle.moe_layer(x32, wl.qtype, prefill_layer.get_blocks, wl.k, logits=logits)
    np.testing.assert_array_equal(buf.ids.cpu().numpy(), ref["ids"])
    _check_layer(buf, buf.out.cpu().numpy(), ref, PREFILL_TOL, T)


@pytest.mark.parametrize("T", [300, 2048])
def test_prefill_not_resident_expert(ctx, prefill_layer, T):
    """An expert whose slot is -1 in the prefill GEMM: reported by id, its
    tokens' outputs NaN, every other token finite.  300 tokens reach the
    tail tiles (at most 64 rows), 2048 the full-tile branch (about 128 rows
    per expert); both groups of a workgroup take the missing-slot exit
    together."""
    wl = prefill_layer.wl
    logits, xbits, x32 = _prefill_inputs(wl, T)
    ids = oracle.topk_select(logits, wl.k)
    counts = np.bincount(ids.reshape(-1), minlength=wl.E)
    victim = int(np.argmax(counts))
    note(f"prefill not-resident T={T}: expert {victim} with {counts[victim]} pairs")
    table = prefill_layer.slot_table.clone()
    table[victim] = -1
    from gpu_util import bf16_tensor
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV, mode=L.MODE_PREFILL,
                             x_dtype=L.DTYPE_BF16)
    out = layer.forward(ctx, buf, prefill_layer.pool.base(), prefill_layer.pool.slot_bytes,
                        prefill_layer.pool.n_slots, table, bf16_tensor(xbits), logits_in=dev(logits)).cpu().numpy()
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_ctx_check(ctx)
    assert ei.value.name == "MOE_ERR_NOT_RESIDENT" and f"expert {victim}" in str(ei.value)
    moe.moe_ctx_check(ctx)
    uses = (ids == victim).any(axis=1)
    assert np.isnan(out[uses]).all(axis=1).all()
    assert np.isfinite(out[~uses]).all()


@pytest.mark.parametrize("case", ["decode-four-calls", "decode-one-call", "prefill-fp32"])
def test_valu_ffn_paths(ctx, decode_layer, prefill_layer, case):
    """Shapes the tuned kernels do not take run the VALU kernels: decode
    batches of more than 1024 pairs (150 tokens x top-8), through the four
    calls and through moe_decode_layer, and prefill with fp32 activations.
    They accumulate in fp32 on fp32 activations, so the decode tolerance
    applies."""
    note(f"VALU FFN path {case}")
    if case.startswith("decode"):
        rl, T = decode_layer, 150
        wl = rl.wl
        x, wr = gi.activations(wl, T), gi.router_weight(wl, 0)
        buf, out = _run_layer(ctx, rl, T, x, wr, fused="layer" if case == "decode-one-call" else False)
        ref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, router_w=wr)
        _check_layer(buf, out, ref, DECODE_TOL, T, lambda lo: oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k,
                                                                                 logits=lo))
    else:
        rl, T = prefill_layer, 300
        wl = rl.wl
        logits, _, x32 = _prefill_inputs(wl, T)
        buf, out = _run_layer(ctx, rl, T, x32, logits=logits, mode=L.MODE_PREFILL, x_dtype=L.DTYPE_F32)
        ref = oracle.moe_layer(x32, wl.qtype, rl.get_blocks, wl.k, logits=logits)
        np.testing.assert_array_equal(buf.ids.cpu().numpy(), ref["ids"])
        _check_layer(buf, out, ref, DECODE_TOL, T)


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_expert_mask_skips_experts(ctx, prefill_layer, mode):
    """Experts masked out are not computed: their y rows keep what they held;
    the others equal an unmasked run bit for bit."""
    wl = prefill_layer.wl
    T = 300 if mode == "prefill" else 4
    note(f"expert mask {mode} T={T}")
    logits, xbits, x32 = _prefill_inputs(wl, T)
    from gpu_util import bf16_tensor
    if mode == "prefill":
        m, xdt, xd = L.MODE_PREFILL, L.DTYPE_BF16, bf16_tensor(xbits)
    else:
        m, xdt, xd = L.MODE_DECODE, L.DTYPE_F32, dev(x32)
    rl = prefill_layer
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV, mode=m, x_dtype=xdt)
    args = (ctx, buf, rl.pool.base(), rl.pool.slot_bytes, rl.pool.n_slots, rl.slot_table, xd)
    layer.forward(*args, logits_in=dev(logits), steps=("route", "permute", "ffn"))
    full = buf.y.cpu().numpy().reshape(T * wl.k, wl.H)
    mask = (np.arange(wl.E) % 3 != 1).astype(np.int32)
    buf.y.fill_(7.0)
    layer.forward(*args, expert_mask=dev(mask), steps=("ffn",))
    torch.cuda.synchronize()
    moe.moe_ctx_check(ctx)
    y = buf.y.cpu().numpy().reshape(T * wl.k, wl.H)
    keep = mask[buf.ids.cpu().numpy().reshape(-1)] == 1
    assert (~keep).any() and keep.any()
    assert (y[~keep] == 7.0).all()
    np.testing.assert_array_equal(y[keep], full[keep])


def _layer_outputs(ctx, rl, T, x, wr, b, lg, fused):
    wl = rl.wl
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV)
    for name in ("logits", "w", "y", "out"):
        getattr(buf, name).fill_(float("nan"))
    for name in ("ids", "offsets", "sorted_pairs", "pair_pos", "active"):
        getattr(buf, name).fill_(-7)
    layer.forward(ctx, buf, rl.pool.base(), rl.pool.slot_bytes, rl.pool.n_slots, rl.slot_table, dev(x),
                  router_w=None if wr is None else dev(wr), bias=None if b is None else dev(b),
                  logits_in=None if lg is None else dev(lg), fused=fused)
    torch.cuda.synchronize()
    moe.moe_ctx_check(ctx)
    return buf, {n: getattr(buf, n).cpu().numpy() for n in
                 ("logits", "ids", "w", "offsets", "sorted_pairs", "pair_pos", "active", "y", "out")}


@pytest.mark.parametrize("case", ["decode-1", "decode-4", "decode-16", "decode-given-2", "wide-1", "wide-64",
                                  "tiny-4"])
def test_decode_layer_equals_two_calls(ctx, decode_layer, wide_layer, case):
    """moe_decode_layer (routing inside the gate/up kernel for T*k <= 64, else
    the two calls) gives bit-identical routing results and outputs to
    moe_route_permute + moe_expert_ffn, and matches the oracle."""
    name, T = case.rsplit("-", 1)
    T = int(T)
    note(f"decode layer {case}")
    rl = {"decode": decode_layer, "decode-given": decode_layer, "wide": wide_layer}.get(name)
    if name == "tiny":
        rl = ResidentLayer(gi.workload("tiny_q8_0"))
    wl = rl.wl
    x = gi.activations(wl, T)
    wr, b, lg = gi.router_weight(wl, 0), gi.router_bias(wl), None
    if name == "decode-given":
        rng = np.random.default_rng(3)
        wr, lg, b = None, rng.standard_normal((T, wl.E)).astype(np.float32), \
            (rng.standard_normal(wl.E) * 0.5).astype(np.float32)
    _, two = _layer_outputs(ctx, rl, T, x, wr, b, lg, True)
    for rep in range(2):
        buf, one = _layer_outputs(ctx, rl, T, x, wr, b, lg, "layer")
        for key in two:
            np.testing.assert_array_equal(one[key], two[key], err_msg=f"{key} (call {rep})")
    if lg is None:
        ref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, router_w=wr, bias=b)
    else:  # the library adds the bias to given logits (in fp32) before selecting
        ref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, logits=(lg + b).astype(np.float32))
    _check_layer(buf, one["out"], ref, DECODE_TOL, T, lambda lo: oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, logits=lo))


def _tie_logits(E):
    """Four tokens of router logits built to stress the selection order:
    small integers (many exact ties, a NaN, a -inf); a row whose top values
    are +0 and -0; a row of one value; ten equal maxima straddling the k-th
    place."""
    rng = np.random.default_rng(4)
    lg = rng.integers(-3, 4, size=(4, E)).astype(np.float32)
    lg[0, 5], lg[0, 20] = np.nan, -np.inf
    lg[1] = -1.0
    lg[1, 3:43:4] = np.array([0.0, -0.0] * 5, dtype=np.float32)
    lg[2] = 0.5
    lg[3] = rng.standard_normal(E).astype(np.float32)
    lg[3, 7:107:10] = 4.0
    return lg


@pytest.mark.parametrize("T", [1, 4])
def test_decode_layer_selection_ties(ctx, decode_layer, T):
    """In-kernel routing on logits with exact ties, signed zeros, NaN and
    -inf: ids equal the oracle's (logit desc, id asc) order exactly, and
    every routing result is bit-identical to the two-call path."""
    rl, wl = decode_layer, decode_layer.wl
    x = gi.activations(wl, T)
    lg = _tie_logits(wl.E)[:T].copy()
    _, two = _layer_outputs(ctx, rl, T, x, None, None, lg, True)
    buf, one = _layer_outputs(ctx, rl, T, x, None, None, lg, "layer")
    for key in two:
        np.testing.assert_array_equal(one[key], two[key], err_msg=key)
    np.testing.assert_array_equal(one["ids"], oracle.topk_select(lg, wl.k))  # NaN reads as -inf on both sides
    ref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, logits=lg)
    np.testing.assert_allclose(one["w"], ref["w"], rtol=1e-5, atol=1e-7)
    assert max_rel_err(one["out"], ref["out"]) <= DECODE_TOL


def test_decode_layer_selection_fallback(ctx, wide_layer):
    """512 experts with every logit equal, and 300 equal maxima: more
    candidates than the threshold selection holds, so the in-kernel routing
    falls back to arg-max rounds; still the oracle's ids and bit-identical
    to the two-call path."""
    rl, wl = wide_layer, wide_layer.wl
    T = 2
    x = gi.activations(wl, T)
    lg = np.zeros((T, wl.E), dtype=np.float32)
    lg[1] = -1.0
    lg[1, np.random.default_rng(9).permutation(wl.E)[:300]] = 0.5
    _, two = _layer_outputs(ctx, rl, T, x, None, None, lg, True)
    _, one = _layer_outputs(ctx, rl, T, x, None, None, lg, "layer")
    for key in two:
        np.testing.assert_array_equal(one[key], two[key], err_msg=key)
    np.testing.assert_array_equal(one["ids"], oracle.topk_select(lg, wl.k))
    ref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, logits=lg)
    assert max_rel_err(one["out"], ref["out"]) <= DECODE_TOL


def test_decode_layer_many_launches_and_graph(ctx, decode_layer):
    """moe_decode_layer called many times in a row on one stream, then the
    same calls captured in a HIP graph and replayed (with eager calls between
    the replays), gives results bit-identical to the two-call path on the
    same inputs every time: no state of one call leaks into the next."""
    rl, wl = decode_layer, decode_layer.wl
    note("decode layer: 6 inputs x 4 eager rounds, then 3 graph replays")
    x0 = gi.activations(wl, 1)
    xs = [np.roll(x0, 97 * i, axis=1).copy() for i in range(6)]
    bias = gi.router_bias(wl)
    wr, b = dev(gi.router_weight(wl, 0)), None if bias is None else dev(bias)
    keys = ("logits", "ids", "w", "offsets", "sorted_pairs", "pair_pos", "active", "y", "out")

    def run(buf, x, fused, stream=None):
        layer.forward(ctx, buf, rl.pool.base(), rl.pool.slot_bytes, rl.pool.n_slots, rl.slot_table, x,
                      router_w=wr, bias=b, fused=fused, stream=stream)

    def new_buf():
        return layer.LayerBuffers(1, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV)

    def poison(buf):
        for name in ("logits", "w", "y", "out"):
            getattr(buf, name).fill_(float("nan"))
        for name in ("ids", "offsets", "sorted_pairs", "pair_pos", "active"):
            getattr(buf, name).fill_(-7)

    xd = [dev(x) for x in xs]
    refs = []
    for x in xd:
        rb = new_buf()
        poison(rb)
        run(rb, x, True)
        torch.cuda.synchronize()
        refs.append({n: getattr(rb, n).cpu().numpy() for n in keys})
    assert len({tuple(r["ids"].reshape(-1)) for r in refs}) > 1  # the inputs route differently
    bufs = [new_buf() for _ in xd]

    def check(tag):
        torch.cuda.synchronize()
        moe.moe_ctx_check(ctx)
        for i, (bb, ref) in enumerate(zip(bufs, refs)):
            for n in keys:
                np.testing.assert_array_equal(getattr(bb, n).cpu().numpy(), ref[n], err_msg=f"{tag} input {i} {n}")

    for rnd in range(4):
        for bb in bufs:
            poison(bb)
        for bb, x in zip(bufs, xd):
            run(bb, x, "layer")
        check(f"eager round {rnd}")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for bb, x in zip(bufs, xd):
            run(bb, x, "layer")
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for bb, x in zip(bufs, xd):
            run(bb, x, "layer")
    extra = new_buf()
    for rep in range(3):
        for bb in bufs:
            poison(bb)
        torch.cuda.synchronize()
        g.replay()
        check(f"graph replay {rep}")
        run(extra, xd[rep], "layer")  # eager launches between replays
        torch.cuda.synchronize()
        np.testing.assert_array_equal(extra.out.cpu().numpy(), refs[rep]["out"])
