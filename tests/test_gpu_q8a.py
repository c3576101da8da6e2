"""Decode with int8 activations (MOE_MODE_DECODE_Q8A, the fork README's W4A8
decode scheme) on the GPU: against the oracle's int8-activation FFN
(oracle.moe_layer(..., act_q8=True)) within 1e-3, and against the float
oracle within the looser 2e-2 that 8-bit activations allow; one call equals
the two-call path bit for bit; the refused cases."""
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

Q8A_TOL = 1e-3    # against the int8-activation oracle: fp32 block sums, and a rare h code
                  # rounded the other way because the two sides' h differ in the last bits
FLOAT_TOL = 2e-2  # against the float oracle: the error of 8-bit activations


@pytest.fixture(scope="module")
def ctx():
    c = moe.Ctx(0)
    yield c
    c.close()


@pytest.fixture(scope="module")
def layers():
    return {"decode": ResidentLayer(gi.workload("decode_q8_0_h2048_e128"), layer_idx=0),
            "wide": ResidentLayer(gi.workload("wide_q4_0_h2048_e512"), layer_idx=0)}


def _run(ctx, rl, T, x, wr, b, fused):
    wl = rl.wl
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV, mode=L.MODE_DECODE_Q8A)
    for name in ("logits", "w", "y", "out"):
        getattr(buf, name).fill_(float("nan"))
    for name in ("ids", "offsets", "sorted_pairs", "pair_pos", "active"):
        getattr(buf, name).fill_(-7)
    layer.forward(ctx, buf, rl.pool.base(), rl.pool.slot_bytes, rl.pool.n_slots, rl.slot_table, dev(x),
                  router_w=dev(wr), bias=None if b is None else dev(b), fused=fused)
    torch.cuda.synchronize()
    moe.moe_ctx_check(ctx)
    return buf, {n: getattr(buf, n).cpu().numpy() for n in ("logits", "ids", "w", "offsets", "sorted_pairs",
                                                           "pair_pos", "active", "y", "out")}


@pytest.mark.parametrize("case", ["decode-1", "decode-4", "decode-16", "decode-100", "wide-1", "wide-64"])
def test_q8a_layer(ctx, layers, case):
    name, T = case.split("-")
    T = int(T)
    rl = layers[name]
    wl = rl.wl
    note(f"int8-activation decode {wl.name} T={T}")
    x, wr, b = gi.activations(wl, T), gi.router_weight(wl, 0), gi.router_bias(wl)
    _, two = _run(ctx, rl, T, x, wr, b, True)
    buf, one = _run(ctx, rl, T, x, wr, b, "layer")
    for key in two:
        np.testing.assert_array_equal(one[key], two[key], err_msg=key)
    ref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, router_w=wr, bias=b, act_q8=True)
    check_routed_layer(one["ids"], one["w"], one["logits"], one["y"], one["out"], ref, Q8A_TOL, T,
                       lambda lo: oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, logits=lo, act_q8=True))
    fref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, logits=one["logits"][:T].astype(np.float64))
    e = max_rel_err(one["out"][:T], fref["out"])
    note(f"   against the float oracle: out max rel err {e:.2e}")
    assert e <= FLOAT_TOL
