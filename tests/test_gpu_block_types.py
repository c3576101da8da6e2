"""The other standard block types (Q4_1, Q5_0, Q5_1) and the K-quants Q4_K,
Q5_K on the GPU: exact dequantisation, and decode (GEMV) and prefill (bf16 MFMA)
layers against the oracle, through the same entry points as Q4_0 / Q8_0."""
import numpy as np
import pytest
import torch

import expert_offload_amd as moe
from expert_offload_amd import _lib as L
from expert_offload_amd import layer
from gen import inputs as gi
import oracle

from gpu_util import DEV, ResidentLayer, bf16_tensor, check_routed_layer, dev, max_rel_err, note

pytestmark = pytest.mark.gpu

TYPES = ["q4_1", "q5_0", "q5_1", "q4_k", "q5_k"]
DECODE_TOL, PREFILL_TOL = 1e-3, 2e-2
QUANT = {"q4_1": gi.quantize_q4_1, "q5_0": gi.quantize_q5_0, "q5_1": gi.quantize_q5_1, "q4_k": gi.quantize_q4_k,
         "q5_k": gi.quantize_q5_k}


@pytest.fixture(scope="module")
def ctx():
    c = moe.Ctx(0)
    yield c
    c.close()


def test_dequantize_q4_k_hand_superblock(ctx):
    """The hand-built Q4_K super-block of the oracle's pins through the
    library's packer and device decoding: the weights worked out by hand."""
    from test_oracle_pins import _golden_q4_k, _hand_superblock_q4_k
    blk = _hand_superblock_q4_k().reshape(1, 1, 144)
    packed = np.empty(144, dtype=np.uint8)
    moe.moe_pack_matrix(L.QTYPE["q4_k"], 1, 256, blk, packed)
    out = torch.full((1, 256), float("nan"), dtype=torch.float32, device=DEV)
    moe.moe_dequantize(ctx, L.QTYPE["q4_k"], dev(packed), 1, 256, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0]
    for item in _golden_q4_k()["weights"]:
        idx, val = item.split(":")
        assert got[int(idx)] == float(val), (idx, got[int(idx)], val)
    np.testing.assert_array_equal(got, oracle.dequant("q4_k", blk)[0].astype(np.float32))


def test_dequantize_q5_k_hand_superblock(ctx):
    """The hand-built Q5_K super-block of the oracle's pins (fifth bits set
    and clear) through the library's packer and device decoding."""
    from test_oracle_pins import _golden_q5_k, _hand_superblock_q5_k
    blk = _hand_superblock_q5_k().reshape(1, 1, 176)
    packed = np.empty(176, dtype=np.uint8)
    moe.moe_pack_matrix(L.QTYPE["q5_k"], 1, 256, blk, packed)
    out = torch.full((1, 256), float("nan"), dtype=torch.float32, device=DEV)
    moe.moe_dequantize(ctx, L.QTYPE["q5_k"], dev(packed), 1, 256, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0]
    for item in _golden_q5_k()["weights"]:
        idx, val = item.split(":")
        assert got[int(idx)] == float(val), (idx, got[int(idx)], val)
    np.testing.assert_array_equal(got, oracle.dequant("q5_k", blk)[0].astype(np.float32))


@pytest.mark.parametrize("qt", TYPES)
@pytest.mark.parametrize("rows,cols", [(3, 256), (17, 768), (64, 2048)])
def test_dequantize_exact(ctx, qt, rows, cols):
    """fp32 output equals the exact weight rounded once to fp32 (d*q is
    exact; d*q + m rounds once, as the format's definition does); bf16 is
    round-to-nearest-even of that fp32."""
    note(f"dequant {qt} {rows}x{cols}")
    rng = np.random.default_rng(rows * cols + 1)
    w = (rng.standard_normal((rows, cols)) * rng.choice([1e-3, 0.02, 3.0, 500.0], (rows, 1)))
    blocks = QUANT[qt](w.astype(np.float32))
    blocks[0, 0, 0:2] = [0, 0]          # d = 0
    blocks[-1, -1, 0:2] = [0x01, 0x00]  # subnormal d
    packed = np.empty(blocks.size, dtype=np.uint8)
    moe.moe_pack_matrix(L.QTYPE[qt], rows, cols, blocks, packed)
    pd = dev(packed)
    out32 = torch.full((rows, cols), float("nan"), dtype=torch.float32, device=DEV)
    out16 = torch.zeros((rows, cols), dtype=torch.bfloat16, device=DEV)
    moe.moe_dequantize(ctx, L.QTYPE[qt], pd, rows, cols, out32)
    moe.moe_dequantize(ctx, L.QTYPE[qt], pd, rows, cols, out16)
    torch.cuda.synchronize()
    ref32 = oracle.dequant(qt, blocks).astype(np.float32)
    got32 = out32.cpu().numpy()
    np.testing.assert_array_equal(got32, ref32)
    got16 = out16.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got16, gi.f32_to_bf16_bits(ref32))


def _workload(qt, idx):
    return gi.Workload(30 + idx, f"decode_{qt}_h2048_e32", H=2048, E=32, k=4, I=768, qtype=qt, batches=(1, 4))


@pytest.fixture(scope="module", params=TYPES)
def typed_layer(request):
    return ResidentLayer(_workload(request.param, TYPES.index(request.param)), layer_idx=0)


def _outputs(ctx, rl, T, x, wr, fused):
    wl = rl.wl
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV)
    for name in ("w", "y", "out"):
        getattr(buf, name).fill_(float("nan"))
    layer.forward(ctx, buf, rl.pool.base(), rl.pool.slot_bytes, rl.pool.n_slots, rl.slot_table, dev(x),
                  router_w=dev(wr), fused=fused)
    torch.cuda.synchronize()
    moe.moe_ctx_check(ctx)
    return {n: getattr(buf, n).cpu().numpy() for n in ("logits", "ids", "w", "y", "out")}


@pytest.mark.parametrize("T", [1, 4, 16])
def test_decode_layer(ctx, typed_layer, T):
    """One call (routing inside the gate/up kernel) equals the two-call path
    bit for bit and the oracle within the decode tolerance."""
    rl, wl = typed_layer, typed_layer.wl
    note(f"decode {wl.qtype} T={T}")
    x, wr = gi.activations(wl, T), gi.router_weight(wl, 0)
    two = _outputs(ctx, rl, T, x, wr, True)
    one = _outputs(ctx, rl, T, x, wr, "layer")
    for key in two:
        np.testing.assert_array_equal(one[key], two[key], err_msg=key)
    ref = oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, router_w=wr)
    check_routed_layer(one["ids"], one["w"], one["logits"], one["y"], one["out"], ref, DECODE_TOL, T,
                       lambda lo: oracle.moe_layer(x, wl.qtype, rl.get_blocks, wl.k, logits=lo))


@pytest.mark.parametrize("T", [37, 300])
def test_prefill_layer(ctx, typed_layer, T):
    """The bf16 MFMA grouped GEMM on these blocks against the oracle."""
    rl, wl = typed_layer, typed_layer.wl
    note(f"prefill {wl.qtype} T={T}")
    rng = np.random.default_rng(T)
    logits = rng.standard_normal((T, wl.E)).astype(np.float32)
    xbits = gi.f32_to_bf16_bits(rng.standard_normal((T, wl.H)).astype(np.float32))
    x32 = gi.bf16_bits_to_f32(xbits)
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device=DEV, mode=L.MODE_PREFILL,
                             x_dtype=L.DTYPE_BF16)
    buf.out.fill_(float("nan"))
    out = layer.forward(ctx, buf, rl.pool.base(), rl.pool.slot_bytes, rl.pool.n_slots, rl.slot_table,
                        bf16_tensor(xbits), logits_in=dev(logits)).cpu().numpy()
    moe.moe_ctx_check(ctx)
    ref = oracle.moe_layer(x32, wl.qtype, rl.get_blocks, wl.k, logits=logits)
    np.testing.assert_array_equal(buf.ids.cpu().numpy(), ref["ids"])
    err = max_rel_err(out, ref["out"])
    note(f"   out max rel err {err:.2e}")
    assert err <= PREFILL_TOL
