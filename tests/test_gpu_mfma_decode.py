"""Decode batches whose experts have many tokens: the experts with at least 8
pairs run on the fp32 matrix cores (ffn_gateup_mfma / ffn_down_mfma), the
rest on the GEMV kernels, and the combine joins them.  Routing is given so
that chosen experts get exactly 7, 8, 9, 16, 17 and 33 pairs (both sides of
the threshold, tiles of 16 pairs with and without a ragged tail), for Q8_0
and Q4_0; outputs against the oracle within the decode tolerance, the one-
and two-call layers bit-identical, and a slot of -1 on a matrix-core expert
reported and NaN-filled."""
import numpy as np
import pytest
import torch

import expert_offload_amd as moe
from expert_offload_amd import layer
from gen import inputs as gi
import oracle

from gpu_util import DEV, ResidentLayer, dev, max_rel_err, note

pytestmark = pytest.mark.gpu

DECODE_TOL = 1e-3
COUNTS = {0: 33, 1: 17, 2: 16, 3: 9, 4: 8, 5: 7}  # pairs per expert; the rest are spread


@pytest.fixture(scope="module")
def ctx():
    c = moe.Ctx(0)
    yield c
    c.close()


def _workload(qt, idx):
    return gi.Workload(50 + idx, f"mfma_{qt}_h512_e16", H=512, E=16, k=2, I=256, qtype=qt, batches=(64,))


@pytest.fixture(scope="module", params=["q8_0", "q4_0"])
def mlayer(request):
    return ResidentLayer(_workload(request.param, ["q8_0", "q4_0"].index(request.param)))


def _logits(T, E, k):
    """Router logits giving expert e exactly COUNTS[e] of the T*k pairs (top-2
    per token with a clear margin); the remaining pairs go to experts 6..15."""
    assert k == 2
    want = []
    for e, n in COUNTS.items():
        want += [e] * n
    rest = T * k - len(want)
    want += [6 + i % (E - 6) for i in range(rest)]
    # sorted by expert, token t takes entries t and t + T: no expert has
    # more than T entries, so a token never names one expert twice
    want.sort()
    firsts, seconds = want[:T], want[T:]
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    for t in range(T):
        a, b = firsts[t], seconds[t]
        assert a != b
        lg[t, a], lg[t, b] = 9.0 + rng.random(), 7.0 + rng.random()
    return lg


def _run(ctx, rl, T, x, lg, fused, table=None):
    wl = rl.wl
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV)
    for name in ("w", "y", "out"):
        getattr(buf, name).fill_(float("nan"))
    layer.forward(ctx, buf, rl.pool.base(), rl.pool.slot_bytes, rl.pool.n_slots,
                  rl.slot_table if table is None else table, dev(x), logits_in=dev(lg), fused=fused)
    torch.cuda.synchronize()
    return buf, {n: getattr(buf, n).cpu().numpy() for n in ("ids", "w", "y", "out")}


def test_mfma_experts_match_oracle(ctx, mlayer):
    wl = mlayer.wl
    T = 64
    note(f"matrix-core decode {wl.qtype}: {T} tokens, experts with {sorted(COUNTS.values())} pairs")
    x, lg = gi.activations(wl, T), _logits(T, wl.E, wl.k)
    counts = np.bincount(oracle.topk_select(lg, wl.k).reshape(-1), minlength=wl.E)
    for e, n in COUNTS.items():
        assert counts[e] == n, (e, counts[e], n)
    moe.moe_ctx_set_timing(ctx, True)
    _, two = _run(ctx, mlayer, T, x, lg, True)
    n_mfma = moe.moe_ctx_kernel_time(ctx, "ffn_gateup_mfma")[0]
    moe.moe_ctx_set_timing(ctx, False)
    moe.moe_ctx_check(ctx)
    assert n_mfma == 1  # the matrix-core kernels ran
    _, one = _run(ctx, mlayer, T, x, lg, "layer")
    moe.moe_ctx_check(ctx)
    for key in two:
        np.testing.assert_array_equal(one[key], two[key], err_msg=key)
    ref = oracle.moe_layer(x, wl.qtype, mlayer.get_blocks, wl.k, logits=lg)
    np.testing.assert_array_equal(two["ids"], ref["ids"])
    ey, eo = max_rel_err(two["y"], ref["y_pairs"]), max_rel_err(two["out"], ref["out"])
    note(f"   y max rel err {ey:.2e}, out max rel err {eo:.2e}")
    assert ey <= DECODE_TOL and eo <= DECODE_TOL
    # per expert: the matrix-core experts' rows on their own
    ids = two["ids"].reshape(-1)
    for e in COUNTS:
        rows = np.nonzero(ids == e)[0]
        assert max_rel_err(two["y"][rows], ref["y_pairs"][rows]) <= DECODE_TOL, e


def test_mfma_expert_without_slot(ctx, mlayer):
    wl = mlayer.wl
    T = 64
    x, lg = gi.activations(wl, T), _logits(T, wl.E, wl.k)
    table = mlayer.slot_table.clone()
    table[1] = -1  # 17 pairs: a matrix-core expert
    _, got = _run(ctx, mlayer, T, x, lg, True, table=table)
    with pytest.raises(moe.MoeError, match="expert 1 "):
        moe.moe_ctx_check(ctx)
    ids = got["ids"].reshape(-1)
    rows = np.nonzero(ids == 1)[0]
    assert np.isnan(got["y"][rows]).all()
    others = np.nonzero(ids != 1)[0]
    assert not np.isnan(got["y"][others]).any()


def test_mfma_layer_graph_replays(ctx, mlayer):
    """The 64-token layer with matrix-core experts, whose kernels the library
    forks onto its side stream and joins back within the call, captured as a
    HIP graph (the fork and join become graph edges): every replay, with the
    outputs poisoned before it and an eager call after it, equals the eager
    call bit for bit."""
    wl = mlayer.wl
    T = 64
    x, lg = dev(gi.activations(wl, T)), dev(_logits(T, wl.E, wl.k))
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV)

    def run():
        layer.forward(ctx, buf, mlayer.pool.base(), mlayer.pool.slot_bytes, mlayer.pool.n_slots, mlayer.slot_table,
                      x, logits_in=lg, fused="layer")

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    s.synchronize()
    moe.moe_ctx_check(ctx)
    names = ("ids", "w", "y", "out")
    eager = {n: getattr(buf, n).clone() for n in names}
    assert not torch.isnan(eager["out"]).any()
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
        for n in names:
            assert torch.equal(getattr(buf, n), eager[n]), f"replay {rep}: {n} differs from the eager call"
        run()
        torch.cuda.synchronize()
        assert torch.equal(buf.out, eager["out"])
