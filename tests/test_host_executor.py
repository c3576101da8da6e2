"""The host executor of the expert FFN (moe_host_expert_ffn, the CPU side of
CPU-GPU co-execution) on the CPU: from packed slot bytes it gives the
oracle's SwiGLU FFN, with AVX-512 and with plain C++, for one and several
tokens and any thread count."""
import numpy as np
import pytest

import expert_offload_amd as moe
from expert_offload_amd import _lib as L
from expert_offload_amd import layer
from gen import inputs as gi
import oracle

TOL = 1e-5  # fp32 accumulation over <= 2048 terms against fp64


def _max_rel(got, ref):
    return float(np.abs(got - ref).max() / np.abs(ref).max())


CASES = [
    gi.Workload(21, "host_q8_0", H=256, E=2, k=1, I=512, qtype="q8_0", batches=(3,)),
    gi.Workload(22, "host_q4_0", H=512, E=2, k=1, I=256, qtype="q4_0", batches=(3,)),
    gi.Workload(23, "host_q4_0_wide", H=2048, E=2, k=1, I=768, qtype="q4_0", batches=(2,)),
    gi.Workload(24, "host_q4_1", H=512, E=2, k=1, I=256, qtype="q4_1", batches=(3,)),
    gi.Workload(25, "host_q5_0", H=256, E=2, k=1, I=512, qtype="q5_0", batches=(2,)),
    gi.Workload(26, "host_q5_1", H=512, E=2, k=1, I=768, qtype="q5_1", batches=(3,)),
    gi.Workload(27, "host_q4_k", H=512, E=2, k=1, I=768, qtype="q4_k", batches=(3,)),
    gi.Workload(28, "host_q5_k", H=512, E=2, k=1, I=768, qtype="q5_k", batches=(3,)),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("vector", [True, False])
def test_host_ffn_matches_oracle(wl, vector):
    if vector and not moe.moe_host_has_avx512():
        pytest.skip("no AVX-512 on this CPU")
    gb, ub, db = gi.expert_blocks(wl, 0, 1)
    slot = layer.pack_expert(wl.qtype, wl.H, wl.I, gb, ub, db)
    n = wl.batches[0]
    x = gi.activations(wl, n)
    ref = oracle.expert_ffn(x, oracle.dequant(wl.qtype, gb), oracle.dequant(wl.qtype, ub),
                            oracle.dequant(wl.qtype, db))
    for threads in (1, 3, 0):
        y = np.full((n, wl.H), np.nan, dtype=np.float32)
        moe.moe_host_expert_ffn(L.QTYPE[wl.qtype], wl.H, wl.I, slot, x, y, threads=threads, vector=vector)
        assert _max_rel(y, ref) <= TOL, (threads, _max_rel(y, ref))
    # one token at a time gives the same rows
    y1 = np.empty((1, wl.H), dtype=np.float32)
    moe.moe_host_expert_ffn(L.QTYPE[wl.qtype], wl.H, wl.I, slot, x[1:2].copy(), y1, vector=vector)
    assert _max_rel(y1[0], ref[1]) <= TOL


def test_host_ffn_vector_equals_plain_within_rounding():
    if not moe.moe_host_has_avx512():
        pytest.skip("no AVX-512 on this CPU")
    wl = CASES[1]
    slot = layer.pack_expert(wl.qtype, wl.H, wl.I, *gi.expert_blocks(wl, 0, 0))
    x = gi.activations(wl, 2)
    a = np.empty((2, wl.H), dtype=np.float32)
    b = np.empty((2, wl.H), dtype=np.float32)
    moe.moe_host_expert_ffn(L.QTYPE[wl.qtype], wl.H, wl.I, slot, x, a, vector=True)
    moe.moe_host_expert_ffn(L.QTYPE[wl.qtype], wl.H, wl.I, slot, x, b, vector=False)
    assert _max_rel(a, b.astype(np.float64)) <= TOL


def test_host_ffn_errors():
    x = np.zeros((1, 256), dtype=np.float32)
    y = np.zeros((1, 256), dtype=np.float32)
    slot = np.zeros(moe.moe_slot_bytes(L.QTYPE["q8_0"], 256, 256), dtype=np.uint8)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_host_expert_ffn(5, 256, 256, slot, x, y)
    assert ei.value.name == "MOE_ERR_UNSUPPORTED_QTYPE"
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_host_expert_ffn(L.QTYPE["q8_0"], 200, 256, slot, x, y)
    assert ei.value.name == "MOE_ERR_INVALID_ARG"
