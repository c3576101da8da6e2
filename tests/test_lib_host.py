"""libmoe on the host (no GPU): the library loads, exports every symbol the
header declares, and its host-only entry points (block-type table, slot
sizes, the ggml -> device layout packer, the bank-type rule, workspace
queries, argument errors) behave as documented."""
import ctypes
import os
import re

import numpy as np
import pytest

import expert_offload_amd as moe
from expert_offload_amd import _lib as L
from gen import inputs as gi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"defined"})


def test_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 20
    lib = moe.lib()
    for n in names:
        assert hasattr(lib, n), f"libmoe does not export {n}"
    assert sorted(moe.EXPORTS) == names


def test_qtype_table():
    assert moe.moe_qtype_info(L.QTYPE["q8_0"]) == (32, 34)
    assert moe.moe_qtype_info(L.QTYPE["q4_0"]) == (32, 18)
    assert moe.moe_qtype_info(L.QTYPE["q4_1"]) == (32, 20)
    assert moe.moe_qtype_info(L.QTYPE["q5_0"]) == (32, 22)
    assert moe.moe_qtype_info(L.QTYPE["q5_1"]) == (32, 24)
    assert moe.moe_qtype_info(L.QTYPE["q4_k"]) == (256, 144)  # one super-block
    assert moe.moe_qtype_info(L.QTYPE["q5_k"]) == (256, 176)
    assert L.QTYPE == {"q4_0": 2, "q4_1": 3, "q5_0": 6, "q5_1": 7, "q8_0": 8, "q4_k": 12,
                       "q5_k": 13}  # ggml's type numbers
    for bad in (0, 1, 4, 5, 9, 10, 11, 14, -1, 99):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_qtype_info(bad)
        assert ei.value.name == "MOE_ERR_UNSUPPORTED_QTYPE"
        assert str(bad) in str(ei.value)


def test_unsupported_qtype_leaves_outputs_untouched():
    a, b = ctypes.c_int(-7), ctypes.c_int(-7)
    rc = moe.lib().moe_qtype_info(14, ctypes.byref(a), ctypes.byref(b))
    assert rc == -2 and a.value == -7 and b.value == -7


@pytest.mark.parametrize("qt,H,I", [("q8_0", 256, 512), ("q8_0", 2048, 768), ("q4_0", 2048, 768),
                                    ("q4_0", 2048, 512), ("q4_0", 4096, 2048), ("q4_1", 2048, 768),
                                    ("q5_0", 2048, 768), ("q5_1", 4096, 2048), ("q4_k", 2048, 768),
                                    ("q5_k", 2048, 768)])
def test_slot_bytes_equal_ggml_bytes(qt, H, I):
    if qt in ("q4_k", "q5_k"):  # 144 / 176 bytes per super-block of 256 weights
        assert moe.moe_slot_bytes(L.QTYPE[qt], H, I) == 3 * H * I // 256 * {"q4_k": 144, "q5_k": 176}[qt]
        return
    per_block = {"q8_0": 34, "q4_0": 18, "q4_1": 20, "q5_0": 22, "q5_1": 24}[qt]
    assert moe.moe_slot_bytes(L.QTYPE[qt], H, I) == 3 * H * I // 32 * per_block


def test_slot_bytes_errors():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_slot_bytes(L.QTYPE["q8_0"], 300, 512)
    assert ei.value.name == "MOE_ERR_INVALID_ARG"
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_slot_bytes(16, 256, 256)
    assert ei.value.name == "MOE_ERR_UNSUPPORTED_QTYPE"


def _unpack_doc_layout(qt, rows, cols, packed):
    """Read the documented device layout back into ggml blocks: per group of
    8 blocks the quant bytes, then the fifth-bit words (Q5_*), the scales d,
    the offsets m (Q4_1, Q5_1); a ggml block is d, [m], [fifth bits], quants."""
    qb = 32 if qt == "q8_0" else 16
    has_m, has_qh = qt in ("q4_1", "q5_1"), qt in ("q5_0", "q5_1")
    bb = gi.BLOCK_BYTES[qt]
    gbytes = 8 * bb
    qh_off, d_off = 8 * qb, 8 * qb + (32 if has_qh else 0)
    m_off = d_off + 16
    out = np.empty((rows, cols // 32, bb), dtype=np.uint8)
    rb = cols // 256 * gbytes
    for r in range(rows):
        for g in range(cols // 256):
            grp = packed[r * rb + g * gbytes: r * rb + (g + 1) * gbytes]
            for b in range(8):
                blk = out[r, 8 * g + b]
                blk[0:2] = grp[d_off + 2 * b: d_off + 2 * b + 2]
                at = 2
                if has_m:
                    blk[2:4] = grp[m_off + 2 * b: m_off + 2 * b + 2]
                    at = 4
                if has_qh:
                    blk[at:at + 4] = grp[qh_off + 4 * b: qh_off + 4 * b + 4]
                    at += 4
                blk[at:] = grp[b * qb:(b + 1) * qb]
    return out


def _unpack_doc_layout_q4_k(rows, cols, packed):
    """Read the documented Q4_K device groups back into ggml super-blocks:
    per group 8 sub-blocks of 16 quant bytes (element j low, j + 16 high in
    byte j), the 12 scale bytes, d, dmin; a ggml super-block is d, dmin,
    scales, then 4 x 32 bytes holding sub-blocks 2i (low) and 2i+1 (high)."""
    out = np.empty((rows, cols // 256, 144), dtype=np.uint8)
    for r in range(rows):
        for g in range(cols // 256):
            grp = packed[(r * (cols // 256) + g) * 144:(r * (cols // 256) + g + 1) * 144]
            sb = out[r, g]
            sb[0:2], sb[2:4], sb[4:16] = grp[140:142], grp[142:144], grp[128:140]
            codes = [[(grp[16 * b + (l % 16)] >> (4 * (l // 16))) & 15 for l in range(32)] for b in range(8)]
            for i in range(4):
                sb[16 + 32 * i:48 + 32 * i] = [codes[2 * i][l] | (codes[2 * i + 1][l] << 4) for l in range(32)]
    return out


def _unpack_doc_layout_q5_k(rows, cols, packed):
    """Read the documented Q5_K device groups back into ggml super-blocks:
    per group 8 sub-blocks of 16 quant bytes (as in Q4_K), their 8 fifth-bit
    words (bit l for element l), the 12 scale bytes, d, dmin; a ggml
    super-block is d, dmin, scales, qh (bit j of byte l for element l of
    sub-block j), then the nibbles as in Q4_K."""
    out = np.empty((rows, cols // 256, 176), dtype=np.uint8)
    for r in range(rows):
        for g in range(cols // 256):
            grp = packed[(r * (cols // 256) + g) * 176:(r * (cols // 256) + g + 1) * 176]
            sb = out[r, g]
            sb[0:2], sb[2:4], sb[4:16] = grp[172:174], grp[174:176], grp[160:172]
            words = [int.from_bytes(bytes(grp[128 + 4 * b:132 + 4 * b]), "little") for b in range(8)]
            sb[16:48] = [sum(((words[j] >> l) & 1) << j for j in range(8)) for l in range(32)]
            codes = [[(grp[16 * b + (l % 16)] >> (4 * (l // 16))) & 15 for l in range(32)] for b in range(8)]
            for i in range(4):
                sb[48 + 32 * i:80 + 32 * i] = [codes[2 * i][l] | (codes[2 * i + 1][l] << 4) for l in range(32)]
    return out


@pytest.mark.parametrize("qt", ["q8_0", "q4_0", "q4_1", "q5_0", "q5_1", "q4_k", "q5_k"])
def test_pack_expert_layout(qt):
    H, I = 512, 256
    rng = np.random.default_rng(1)
    quant = {"q8_0": gi.quantize_q8_0, "q4_0": gi.quantize_q4_0, "q4_1": gi.quantize_q4_1,
             "q5_0": gi.quantize_q5_0, "q5_1": gi.quantize_q5_1, "q4_k": gi.quantize_q4_k,
             "q5_k": gi.quantize_q5_k}[qt]
    unpack = {"q4_k": _unpack_doc_layout_q4_k, "q5_k": _unpack_doc_layout_q5_k}.get(
        qt, lambda r, c, p: _unpack_doc_layout(qt, r, c, p))
    g = quant(rng.standard_normal((I, H)).astype(np.float32))
    u = quant(rng.standard_normal((I, H)).astype(np.float32))
    d = quant(rng.standard_normal((H, I)).astype(np.float32))
    from expert_offload_amd.layer import pack_expert
    packed = pack_expert(qt, H, I, g, u, d)
    n1 = g.size
    assert packed.size == g.size + u.size + d.size
    np.testing.assert_array_equal(unpack(I, H, packed[:n1]), g)
    np.testing.assert_array_equal(unpack(I, H, packed[n1:2 * n1]), u)
    np.testing.assert_array_equal(unpack(H, I, packed[2 * n1:]), d)


def test_pack_expert_small_destination():
    H, I = 256, 256
    g = np.zeros((I, H // 32, 34), np.uint8)
    dst = np.zeros(10, np.uint8)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_pack_expert(8, H, I, g, g, g, dst)
    assert ei.value.name == "MOE_ERR_WORKSPACE"


def test_bank_type_rule():
    q4, q8 = L.QTYPE["q4_0"], L.QTYPE["q8_0"]
    assert moe.moe_check_bank_types([[q4, q4, q4]] * 5) == q4
    mixed = [[q4, q4, q4]] * 5
    mixed[1] = [q4, q4, q8]
    mixed[3] = [q8, q8, q8]
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_check_bank_types(mixed)
    assert ei.value.name == "MOE_ERR_MIXED_QTYPE"
    assert "1, 3" in str(ei.value)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_check_bank_types([[14, 14, 14]])
    assert ei.value.name == "MOE_ERR_UNSUPPORTED_QTYPE"


def test_workspace_queries():
    assert moe.moe_permute_workspace_size(16, 8, 128) == 0
    assert moe.moe_permute_workspace_size(512, 8, 128) == 0  # 4096 pairs: one workgroup
    # 4097..4608 pairs: 9 chunks of 512, counts and bases for 128 experts
    assert moe.moe_permute_workspace_size(4097, 1, 128) == 2 * 9 * 128 * 4
    assert moe.moe_permute_workspace_size(4096, 8, 128) == 2 * 64 * 128 * 4
    args = L.moe_ffn_args(qtype=8, H=2048, I=768, T=16, k=8, E=128, mode=0, x_dtype=0, n_slots=128,
                          slot_bytes=moe.moe_slot_bytes(8, 2048, 768))
    assert moe.moe_expert_ffn_workspace_size(args) >= 16 * 8 * 768 * 4
    bad = L.moe_ffn_args(qtype=14, H=2048, I=768, T=16, k=8, E=128, mode=0, x_dtype=0, slot_bytes=1)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_expert_ffn_workspace_size(bad)
    assert ei.value.name == "MOE_ERR_UNSUPPORTED_QTYPE"


def test_null_context_is_an_error():
    lib = moe.lib()
    assert lib.moe_route(None, None, 0, None, None, None, 1, 256, 8, 2, None, None, None, None) == -1
    assert lib.moe_permute(None, None, 1, 2, 8, None, None, None, None, None, 0, None) == -1
    assert lib.moe_combine(None, None, None, 1, 2, 256, None, None) == -1
    assert lib.moe_ctx_check(None, None) == -1
    assert "ctx is NULL" in moe.moe_last_error()


def test_q8a_mode_refusals():
    """Int8-activation decode: banks of a type without signed codes, and
    batches past 1024 pairs, are refused on the host with the documented
    errors."""
    wl = gi.workload("tiny_q8_0")
    for qt, T, want in (("q4_1", 4, "MOE_ERR_UNSUPPORTED_QTYPE"), ("q4_k", 4, "MOE_ERR_UNSUPPORTED_QTYPE"),
                        ("q8_0", 600, "MOE_ERR_INVALID_ARG")):
        args = L.moe_ffn_args(qtype=L.QTYPE[qt], H=wl.H, I=wl.I, T=T, k=wl.k, E=wl.E, mode=L.MODE_DECODE_Q8A,
                              x_dtype=L.DTYPE_F32, n_slots=1, slot_bytes=moe.moe_slot_bytes(L.QTYPE[qt], wl.H, wl.I))
        with pytest.raises(moe.MoeError) as ei:
            L.moe_expert_ffn_workspace_size(args)
        assert ei.value.name == want, (qt, T, ei.value.name)
    ok = L.moe_ffn_args(qtype=L.QTYPE["q8_0"], H=wl.H, I=wl.I, T=4, k=wl.k, E=wl.E, mode=L.MODE_DECODE_Q8A,
                        x_dtype=L.DTYPE_F32, n_slots=1, slot_bytes=moe.moe_slot_bytes(L.QTYPE["q8_0"], wl.H, wl.I))
    # h rows, then codes, scales and code sums of x and of h
    assert L.moe_expert_ffn_workspace_size(ok) >= 4 * wl.k * wl.I * 4 + 4 * wl.H + 4 * wl.k * wl.I
