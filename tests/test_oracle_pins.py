"""Pins of the CPU oracle against closed forms, brute force and independent
simulations (no GPU).  Each pin is chosen so that a plausible slip in the
oracle (wrong byte or nibble order, dropped -8 offset, transposed router,
wrong tie rule, missing renormalisation, unstable grouping, swapped SwiGLU
operands, wrong combine index, wrong LRU victim) fails at least one test.
"""
import collections
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gen import inputs as gi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.txt")


# ---------------------------------------------------------------- helpers
def fp16_bits_to_float(bits: int) -> float:
    """IEEE binary16 decoded from its fields (independent of NumPy's float16)."""
    sign = -1.0 if bits & 0x8000 else 1.0
    exp = (bits >> 10) & 0x1F
    man = bits & 0x3FF
    if exp == 0:
        return sign * man * 2.0 ** -24
    assert exp != 31, "inf/nan scales are outside the format's use"
    return sign * (1.0 + man / 1024.0) * 2.0 ** (exp - 15)


def build_block(qtype: str, d_bits: int, codes) -> np.ndarray:
    """Pack one block by hand from the format description."""
    codes = list(codes)
    assert len(codes) == 32
    if qtype == "q8_0":
        body = [c & 0xFF for c in codes]
    else:
        body = [(codes[j] & 0xF) | ((codes[j + 16] & 0xF) << 4) for j in range(16)]
    return np.array([d_bits & 0xFF, d_bits >> 8] + body, dtype=np.uint8)


GOLDEN_AFFINE = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks_affine.txt")


def build_block_affine(qtype: str, d_bits: int, m_bits: int, codes) -> np.ndarray:
    """Pack one Q4_1 / Q5_0 / Q5_1 block by hand from the format description."""
    codes = list(codes)
    assert len(codes) == 32
    out = [d_bits & 0xFF, d_bits >> 8]
    if qtype in ("q4_1", "q5_1"):
        out += [m_bits & 0xFF, m_bits >> 8]
    if qtype in ("q5_0", "q5_1"):
        word = 0
        for j, c in enumerate(codes):
            if c & 0x10:
                word |= 1 << j
        out += list(word.to_bytes(4, "little"))
    out += [(codes[j] & 0xF) | ((codes[j + 16] & 0xF) << 4) for j in range(16)]
    return np.array(out, dtype=np.uint8)


def affine_weight(qtype: str, d, m, c):
    """Exact weight from the format description (Fractions)."""
    return d * (c - 16) if qtype == "q5_0" else d * c + m


def load_golden_affine():
    rows = []
    for line in open(GOLDEN_AFFINE):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        qt, dh, dv, mh, mv, codes = [f.strip() for f in line.split(";")]
        rows.append((qt, int(dh, 16), float(dv), None if mh == "-" else int(mh, 16), float(mv),
                     [int(c) for c in codes.split()]))
    return rows


def load_golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        qt, dh, dv, codes = [f.strip() for f in line.split(";")]
        rows.append((qt, int(dh, 16), float(dv), [int(c) for c in codes.split()]))
    return rows


# ---------------------------------------------------------------- dequant
@pytest.mark.parametrize("row", load_golden(), ids=lambda r: f"{r[0]}-{r[1]:04X}")
def test_dequant_hand_blocks(row):
    qt, d_bits, d_val, codes = row
    assert fp16_bits_to_float(d_bits) == d_val  # the fixture's hand-derived d
    blk = build_block(qt, d_bits, codes)[None, None, :]
    got = oracle.dequant(qt, blk)[0]
    off = 0 if qt == "q8_0" else 8
    want = np.array([d_val * (c - off) for c in codes], dtype=np.float64)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("qt", ["q8_0", "q4_0"])
def test_dequant_brute_force_all_codes(qt):
    """Every code value times a set of scales, element position varied."""
    codes_all = list(range(-128, 128)) if qt == "q8_0" else list(range(16))
    d_bits_set = [0x3C00, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0xB555, 0x2E66]
    for d_bits in d_bits_set:
        dv = fp16_bits_to_float(d_bits)
        for start in range(0, len(codes_all), 32):
            chunk = (codes_all[start:start + 32] + codes_all)[:32]
            chunk = chunk[::-1] if (start // 32) % 2 else chunk
            blk = build_block(qt, d_bits, chunk)[None, None, :]
            got = oracle.dequant(qt, blk)[0]
            off = 0 if qt == "q8_0" else 8
            for i, c in enumerate(chunk):
                exact = Fraction(dv) * (c - off)
                assert Fraction(float(got[i])) == exact


@pytest.mark.parametrize("row", load_golden_affine(), ids=lambda r: f"{r[0]}-{r[1]:04X}")
def test_dequant_hand_blocks_affine(row):
    qt, d_bits, d_val, m_bits, m_val, codes = row
    assert fp16_bits_to_float(d_bits) == d_val
    if m_bits is not None:
        assert fp16_bits_to_float(m_bits) == m_val
    blk = build_block_affine(qt, d_bits, m_bits or 0, codes)[None, None, :]
    assert blk.shape[-1] == gi.BLOCK_BYTES[qt]
    got = oracle.dequant(qt, blk)[0]
    for i, c in enumerate(codes):
        assert Fraction(float(got[i])) == affine_weight(qt, Fraction(d_val), Fraction(m_val), c), (i, c)


@pytest.mark.parametrize("qt", ["q4_1", "q5_0", "q5_1"])
def test_dequant_brute_force_all_codes_affine(qt):
    """Every code at every position, a set of scales and offsets."""
    top = 15 if qt == "q4_1" else 31
    d_bits_set = [0x3C00, 0x0001, 0x03FF, 0x7BFF, 0xB555, 0x2E66]
    m_bits_set = [0x0000, 0xC280, 0x7BFF, 0x8001] if qt != "q5_0" else [0]
    for d_bits in d_bits_set:
        for m_bits in m_bits_set:
            dv, mv = Fraction(fp16_bits_to_float(d_bits)), Fraction(fp16_bits_to_float(m_bits))
            for shift in range(0, 32, 5):
                codes = [(j + shift) % (top + 1) for j in range(32)]
                got = oracle.dequant(qt, build_block_affine(qt, d_bits, m_bits, codes)[None, None, :])[0]
                for i, c in enumerate(codes):
                    assert Fraction(float(got[i])) == affine_weight(qt, dv, mv, c)


@pytest.mark.parametrize("qt", ["q4_1", "q5_0", "q5_1"])
def test_quantiser_error_bound_affine(qt):
    """The harness quantisers stay within half a step (plus fp16 rounding of
    the scale) of the fp32 input, decoded by the oracle; Q5_0's code range
    is one step short on the side opposite the largest element, which is
    clipped by up to a full step."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    blocks = {"q4_1": gi.quantize_q4_1, "q5_0": gi.quantize_q5_0, "q5_1": gi.quantize_q5_1}[qt](w)
    got = oracle.dequant(qt, blocks)
    b = w.reshape(8, 8, 32).astype(np.float64)
    if qt == "q5_0":
        bound = np.abs(b).max(axis=2) / 16.0
    else:
        bound = 0.5 * (b.max(axis=2) - b.min(axis=2)) / (15 if qt == "q4_1" else 31)
    err = np.abs(got - w).reshape(8, 8, 32).max(axis=2)
    assert (err <= bound * 1.01 + 2 * np.abs(b).max(axis=2) * 2.0 ** -10).all()


GOLDEN_Q4_K = os.path.join(os.path.dirname(__file__), "golden", "hand_superblock_q4_k.txt")


def _golden_q4_k():
    f = {}
    for line in open(GOLDEN_Q4_K):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split(":", 1)
            f[k.strip()] = v.split()
    return f


def _hand_superblock_q4_k():
    """The golden super-block's bytes, built here from the field rules."""
    f = _golden_q4_k()
    b = [0x00, 0x3C, 0x00, 0x38] + [int(h, 16) for h in f["scales"]]
    for i in range(4):
        b += [((l + i) & 15) | (((3 * l + i) & 15) << 4) for l in range(32)]
    return np.array(b, dtype=np.uint8)


def test_dequant_q4_k_hand_superblock():
    """Hand-built Q4_K super-block: the 6-bit scale and min fields and
    selected weights worked out by hand from the format (golden file)."""
    f = _golden_q4_k()
    blk = _hand_superblock_q4_k()
    sc, mn = oracle.q4_k_scales_mins(blk[4:16])
    assert sc.tolist() == [int(v) for v in f["expected_scales"]]
    assert mn.tolist() == [int(v) for v in f["expected_mins"]]
    got = oracle.dequant("q4_k", blk[None, None, :])[0]
    assert got.shape == (256,)
    for item in f["weights"]:
        idx, val = item.split(":")
        assert got[int(idx)] == float(val), (idx, got[int(idx)], val)


def test_dequant_q4_k_brute_force():
    """Every code at every position of every sub-block, with scale and min
    codes over the full 6-bit range (high bits set and clear), against the
    exact d * scale * q - dmin * min; the super-blocks are packed by the
    harness packer (field rules written independently of the oracle)."""
    rng = np.random.default_rng(13)
    for d_bits, m_bits in [(0x3C00, 0x3800), (0x2E66, 0x0001), (0x7BFF, 0x03FF), (0x0001, 0x7BFF)]:
        dv, mv = Fraction(fp16_bits_to_float(d_bits)), Fraction(fp16_bits_to_float(m_bits))
        for trial in range(6):
            sc = rng.integers(0, 64, 8)
            mn = rng.integers(0, 64, 8)
            sc[trial % 8], mn[(trial + 3) % 8] = 63, 0
            q = (np.arange(256).reshape(8, 32) * (trial + 1) + trial) % 16
            blk = gi.pack_q4_k(np.float32(fp16_bits_to_float(d_bits)), np.float32(fp16_bits_to_float(m_bits)),
                               sc, mn, q)
            assert int(blk[0]) | int(blk[1]) << 8 == d_bits and int(blk[2]) | int(blk[3]) << 8 == m_bits
            got = oracle.dequant("q4_k", blk[None, None, :])[0]
            for j in range(8):
                for l in range(32):
                    want = dv * int(sc[j]) * int(q[j, l]) - mv * int(mn[j])
                    assert Fraction(float(got[32 * j + l])) == want, (j, l)


def test_quantiser_error_bound_q4_k():
    """The harness Q4_K quantiser stays within about a step of its input:
    half a code step plus the 6-bit rounding of scale and min."""
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((6, 512)) * 0.02).astype(np.float32)
    got = oracle.dequant("q4_k", gi.quantize_q4_k(w))
    sb = w.reshape(6, 2, 8, 32).astype(np.float64)
    step = (sb.max(axis=3) - np.minimum(sb.min(axis=3), 0)) / 15
    err = np.abs(got - w).reshape(6, 2, 8, 32).max(axis=3)
    assert (err <= 1.5 * step.max(axis=2)[..., None]).all()


GOLDEN_Q5_K = os.path.join(os.path.dirname(__file__), "golden", "hand_superblock_q5_k.txt")


def _golden_q5_k():
    f = {}
    for line in open(GOLDEN_Q5_K):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split(":", 1)
            f[k.strip()] = v.split()
    return f


def _hand_superblock_q5_k():
    """The golden Q5_K super-block's bytes, built here from the field rules."""
    f = _golden_q5_k()
    b = [0x00, 0x3C, 0x00, 0x38] + [int(h, 16) for h in f["scales"]]
    b += [1 << (l & 7) for l in range(32)]
    for i in range(4):
        b += [((l + i) & 15) | (((3 * l + i) & 15) << 4) for l in range(32)]
    return np.array(b, dtype=np.uint8)


def test_dequant_q5_k_hand_superblock():
    """Hand-built Q5_K super-block: selected weights worked out by hand from
    the format (golden file), fifth bits set and clear."""
    f = _golden_q5_k()
    blk = _hand_superblock_q5_k()
    assert blk.shape == (176,)
    sc, mn = oracle.q4_k_scales_mins(blk[4:16])
    assert sc.tolist() == [int(v) for v in f["expected_scales"]]
    assert mn.tolist() == [int(v) for v in f["expected_mins"]]
    got = oracle.dequant("q5_k", blk[None, None, :])[0]
    assert got.shape == (256,)
    for item in f["weights"]:
        idx, val = item.split(":")
        assert got[int(idx)] == float(val), (idx, got[int(idx)], val)


def test_dequant_q5_k_reduces_to_q4_k():
    """With every fifth bit clear, a Q5_K super-block is the Q4_K one with
    the same scale bytes and nibbles; with every bit set, each weight gains
    16 * d * scale_j (its sub-block's scale)."""
    rng = np.random.default_rng(17)
    k4 = _hand_superblock_q4_k()
    k4[4:16] = rng.integers(0, 256, 12)
    k4[16:] = rng.integers(0, 256, 128)
    k5 = np.concatenate([k4[:16], np.zeros(32, np.uint8), k4[16:]])
    w4 = oracle.dequant("q4_k", k4[None, None, :])[0]
    np.testing.assert_array_equal(oracle.dequant("q5_k", k5[None, None, :])[0], w4)
    k5[16:48] = 0xFF
    sc, _ = oracle.q4_k_scales_mins(k4[4:16])
    want = w4 + np.repeat(16.0 * 1.0 * sc, 32)  # d = 1.0
    np.testing.assert_array_equal(oracle.dequant("q5_k", k5[None, None, :])[0], want)


def test_dequant_q5_k_brute_force():
    """Every code 0..31 at every position of every sub-block, scale and min
    codes over the 6-bit range, against the exact d * scale * q - dmin * min;
    super-blocks packed by the harness packer."""
    rng = np.random.default_rng(19)
    for d_bits, m_bits in [(0x3C00, 0x3800), (0x2E66, 0x0001), (0x7BFF, 0x03FF)]:
        dv, mv = Fraction(fp16_bits_to_float(d_bits)), Fraction(fp16_bits_to_float(m_bits))
        for trial in range(4):
            sc = rng.integers(0, 64, 8)
            mn = rng.integers(0, 64, 8)
            sc[trial % 8], mn[(trial + 5) % 8] = 63, 0
            q = (np.arange(256).reshape(8, 32) * (2 * trial + 1) + trial) % 32
            blk = gi.pack_q5_k(np.float32(fp16_bits_to_float(d_bits)), np.float32(fp16_bits_to_float(m_bits)),
                               sc, mn, q)
            assert blk.shape == (176,)
            got = oracle.dequant("q5_k", blk[None, None, :])[0]
            for j in range(8):
                for l in range(32):
                    want = dv * int(sc[j]) * int(q[j, l]) - mv * int(mn[j])
                    assert Fraction(float(got[32 * j + l])) == want, (j, l)


def test_quantiser_error_bound_q5_k():
    """The harness Q5_K quantiser stays within about a step of its input,
    and about half the Q4_K quantiser's error on the same weights."""
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((6, 512)) * 0.02).astype(np.float32)
    got = oracle.dequant("q5_k", gi.quantize_q5_k(w))
    sb = w.reshape(6, 2, 8, 32).astype(np.float64)
    step = (sb.max(axis=3) - np.minimum(sb.min(axis=3), 0)) / 31
    err = np.abs(got - w).reshape(6, 2, 8, 32).max(axis=3)
    assert (err <= 1.5 * step.max(axis=2)[..., None]).all()
    e4 = np.abs(oracle.dequant("q4_k", gi.quantize_q4_k(w)) - w).mean()
    assert np.abs(got - w).mean() < 0.7 * e4


def test_dequant_layout_rows_and_blocks():
    """Blocks run along the input dimension; rows stack (shape [rows, nblk*32])."""
    rng = np.random.default_rng(3)
    blocks = gi.quantize_q8_0(rng.standard_normal((3, 96)).astype(np.float32))
    w = oracle.dequant_q8_0(blocks)
    assert w.shape == (3, 96)
    for r in range(3):
        for b in range(3):
            d = fp16_bits_to_float(int(blocks[r, b, 0]) | (int(blocks[r, b, 1]) << 8))
            q = blocks[r, b, 2:].view(np.int8).astype(np.float64)
            np.testing.assert_array_equal(w[r, 32 * b:32 * b + 32], d * q)


@pytest.mark.parametrize("qt", ["q8_0", "q4_0"])
def test_round_trip_extreme_code(qt):
    """quantise(dequant(b)) == b for blocks holding the extreme code."""
    rng = np.random.default_rng(7)
    quant = gi.quantize_q8_0 if qt == "q8_0" else gi.quantize_q4_0
    for trial in range(200):
        d_bits = int(rng.integers(0x0400, 0x5800))  # positive normal fp16 scales
        if qt == "q4_0" and trial % 2:
            d_bits |= 0x8000  # negative scales are legal in q4_0
        if qt == "q8_0":
            codes = rng.integers(-127, 128, 32)
            codes[rng.integers(32)] = 127 if trial % 2 else -127
        else:
            codes = rng.integers(1, 16, 32)
            codes[rng.integers(32)] = 0
        blk = build_block(qt, d_bits, codes.tolist())[None, None, :]
        w = oracle.dequant(qt, blk).astype(np.float32)
        again = quant(w)
        np.testing.assert_array_equal(again, blk)


# ---------------------------------------------------------------- router
def test_router_logits_loop():
    rng = np.random.default_rng(11)
    T, H, E = 3, 7, 5
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = rng.standard_normal((E, H)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    got = oracle.router_logits(x, wr, b)
    assert got.shape == (T, E)
    for t in range(T):
        for e in range(E):
            want = math.fsum(float(x[t, h]) * float(wr[e, h]) for h in range(H)) + float(b[e])
            assert abs(got[t, e] - want) <= 1e-12 * (1 + abs(want))


def test_softmax_properties():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((6, 9)) * 4
    p = oracle.softmax(l)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.softmax(l + 123.0), p, rtol=1e-13)
    # closed form on a 2-vector: logistic function
    a = oracle.softmax(np.array([[0.3, -1.2]]))[0, 0]
    assert abs(a - 1.0 / (1.0 + math.exp(-1.5))) < 1e-15


def _brute_topk(row, k):
    """Best k-subset by lexicographic (logit desc, id asc) order, by enumeration."""
    E = len(row)
    keyed = sorted(range(E), key=lambda e: (-float(row[e]), e))
    best = None
    for sub in itertools.combinations(range(E), k):
        # a subset is the top-k iff no outside element beats an inside one
        ok = all((-float(row[o]), o) > (-float(row[i]), i)
                 for o in range(E) if o not in sub for i in sub)
        if ok:
            assert best is None
            best = sub
    assert best is not None
    return sorted(best, key=lambda e: (-float(row[e]), e)), keyed[:k]


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(17)
    for trial in range(60):
        E = int(rng.integers(2, 8))
        k = int(rng.integers(1, E + 1))
        row = rng.integers(-2, 3, E).astype(np.float32)  # many exact ties
        if trial % 3 == 0:
            row = rng.standard_normal(E).astype(np.float32)
        got = oracle.topk_select(row[None, :], k)[0].tolist()
        want, _ = _brute_topk(row, k)
        assert got == want, (row, k)


def test_topk_planted_ties_lower_id_wins():
    l = np.array([[0.5, 2.0, 2.0, -1.0, 2.0, 0.5]], dtype=np.float32)
    assert oracle.topk_select(l, 2)[0].tolist() == [1, 2]
    assert oracle.topk_select(l, 4)[0].tolist() == [1, 2, 4, 0]
    # -0.0 and +0.0 compare equal: lower id first
    z = np.array([[0.0, -0.0, -1.0]], dtype=np.float32)
    z[0, 0] = -0.0
    z[0, 1] = 0.0
    assert oracle.topk_select(z, 2)[0].tolist() == [0, 1]


def test_topk_decides_in_fp32():
    """Two float64 logits that round to one fp32 value tie -> lower id."""
    a = 1.0
    b = 1.0 + 2.0 ** -30  # larger in float64, equal in fp32
    assert np.float32(a) == np.float32(b)
    assert oracle.topk_select(np.array([[a, b]]), 1)[0].tolist() == [0]


def test_topk_gap_brute_force():
    """topk_gap = k-th minus (k+1)-th largest logit, against Python's own
    sort of each row; ties give 0, k = E gives inf."""
    rng = np.random.default_rng(23)
    for trial in range(200):
        E = int(rng.integers(2, 12))
        k = int(rng.integers(1, E + 1))
        row = rng.standard_normal(E)
        if trial % 4 == 0:
            row = rng.integers(-2, 3, E).astype(np.float64)  # exact ties
        desc = sorted(row.tolist(), reverse=True)
        want = math.inf if k == E else desc[k - 1] - desc[k]
        assert oracle.topk_gap(row[None, :], k)[0] == want, (row, k)
    # hand-worked rows
    l = np.array([[1.0, 5.0, 3.0, 4.0], [2.0, 2.0, 1.0, 0.0]])
    assert oracle.topk_gap(l, 1).tolist() == [1.0, 0.0]
    assert oracle.topk_gap(l, 2).tolist() == [1.0, 1.0]
    assert oracle.topk_gap(l, 3).tolist() == [2.0, 1.0]
    assert oracle.topk_gap(l, 4).tolist() == [math.inf, math.inf]


def test_nan_logits_read_as_minus_inf():
    """A NaN logit is never chosen over a number, ties with -inf (lower id
    first) and has probability 0; expected ids and weights worked by hand."""
    nan, inf = float("nan"), float("inf")
    l = np.array([[0.5, nan, 0.25, -inf, 0.25, nan]], dtype=np.float32)
    assert oracle.topk_select(l, 3)[0].tolist() == [0, 2, 4]
    assert oracle.topk_select(l, 6)[0].tolist() == [0, 2, 4, 1, 3, 5]
    ids, w = oracle.route(l, 3)
    e = math.exp(-0.25)  # exp(0.25 - 0.5)
    np.testing.assert_allclose(w[0], [1 / (1 + 2 * e), e / (1 + 2 * e), e / (1 + 2 * e)], rtol=1e-15)
    p = oracle.softmax(l.astype(np.float64))[0]
    assert p[1] == 0.0 and p[3] == 0.0 and p[5] == 0.0
    np.testing.assert_allclose(p.sum(), 1.0, rtol=1e-15)
    # the gap treats NaN as -inf too: 0.25 - (-inf), and two -inf tie at 0
    assert oracle.topk_gap(l, 3)[0] == inf
    assert oracle.topk_gap(l, 4)[0] == 0.0


def test_renormalised_weights():
    rng = np.random.default_rng(19)
    l = rng.standard_normal((50, 16)) * 3
    for k in (1, 3, 8, 16):
        ids, w = oracle.route(l, k)
        np.testing.assert_allclose(w.sum(-1), 1.0, rtol=0, atol=k * 2.0 ** -52 * 4)
        assert np.all(w > 0)
        # weights follow the ids' order: non-increasing
        assert np.all(np.diff(w, axis=-1) <= 1e-15)
    ids, w = oracle.route(l, 16)  # k == E: renormalisation is the softmax itself
    p = oracle.softmax(l)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(int), -1), rtol=1e-14)
    ids, w = oracle.route(l, 1)
    np.testing.assert_array_equal(w, 1.0)
    # closed form for k = 2: w0 = 1 / (1 + exp(l1 - l0))
    ids, w = oracle.route(l, 2)
    r = np.take_along_axis(l, ids.astype(int), -1)
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(r[:, 1] - r[:, 0])), rtol=1e-14)


# ---------------------------------------------------------------- permute
def test_permute_matches_stable_argsort():
    rng = np.random.default_rng(23)
    for T, k, E in [(1, 1, 1), (4, 2, 8), (16, 8, 128), (7, 3, 5), (33, 10, 512)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        off, sp, pos, active = oracle.permute(ids, E)
        flat = ids.ravel()
        np.testing.assert_array_equal(sp, np.argsort(flat, kind="stable"))
        np.testing.assert_array_equal(np.bincount(flat, minlength=E), np.diff(off))
        assert off[0] == 0 and off[-1] == T * k
        np.testing.assert_array_equal(sp[pos], np.arange(T * k))  # inverse map
        np.testing.assert_array_equal(active, np.flatnonzero(np.bincount(flat, minlength=E)))
        data = rng.standard_normal(T * k)
        np.testing.assert_array_equal(data[sp][pos], data)  # gather then scatter


def test_permute_duplicates_stable():
    ids = np.array([[2, 0], [2, 1], [0, 2]], dtype=np.int32)
    off, sp, pos, active = oracle.permute(ids, 3)
    assert off.tolist() == [0, 2, 3, 6]
    assert sp.tolist() == [1, 4, 3, 0, 2, 5]  # p -> e: 0->2 1->0 2->2 3->1 4->0 5->2
    assert active.tolist() == [0, 1, 2]


# ---------------------------------------------------------------- FFN and combine
def _dense_ffn_loops(x, wg, wu, wd):
    """SwiGLU FFN by explicit loops: silu on the gate projection, times up."""
    H, I = wd.shape
    g = [math.fsum(wg[i, h] * x[h] for h in range(H)) for i in range(I)]
    u = [math.fsum(wu[i, h] * x[h] for h in range(H)) for i in range(I)]
    a = [gi_ / (1.0 + math.exp(-gi_)) * ui for gi_, ui in zip(g, u)]
    return np.array([math.fsum(wd[h, i] * a[i] for i in range(I)) for h in range(H)])


def test_silu_special_values():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.silu(np.array([40.0])), 40.0, rtol=1e-15)
    assert abs(oracle.silu(np.array([-40.0]))[0]) < 1e-15
    z = 0.7
    assert abs(oracle.silu(np.array([z]))[0] - z / (1 + math.exp(-z))) < 1e-16


@pytest.mark.parametrize("qt", ["q8_0", "q4_0", "q4_k"])
def test_single_expert_k1_is_dense_ffn(qt):
    """E = 1, k = 1: the layer is the dense SwiGLU FFN of that expert (w = 1)."""
    rng = np.random.default_rng(29)
    H, I, T = (64, 96, 3) if qt != "q4_k" else (256, 256, 2)
    quant = {"q8_0": gi.quantize_q8_0, "q4_0": gi.quantize_q4_0, "q4_k": gi.quantize_q4_k}[qt]
    blocks = (quant((rng.standard_normal((I, H)) * 0.1).astype(np.float32)),
              quant((rng.standard_normal((I, H)) * 0.1).astype(np.float32)),
              quant((rng.standard_normal((H, I)) * 0.1).astype(np.float32)))
    x = rng.standard_normal((T, H)).astype(np.float32)
    res = oracle.moe_layer(x, qt, lambda e: blocks, 1,
                           logits=rng.standard_normal((T, 1)))
    np.testing.assert_array_equal(res["w"], 1.0)
    wg, wu, wd = (oracle.dequant(qt, b) for b in blocks)
    for t in range(T):
        want = _dense_ffn_loops(x[t].astype(np.float64), wg, wu, wd)
        np.testing.assert_allclose(res["out"][t], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("qt", ["q8_0", "q4_0"])
def test_layer_k_above_one_is_per_token_dense_sum(qt):
    """k >= 2: every token's output equals, token by token, the sum over
    its k chosen experts (logit desc, id asc) of exp-weighted dense SwiGLU
    FFNs computed by explicit loops, with the weights worked from the logits
    by math.exp: no grouping, gathering or scattering involved."""
    rng = np.random.default_rng(41)
    H, I, E, k, T = 64, 96, 6, 3, 5
    quant = gi.quantize_q8_0 if qt == "q8_0" else gi.quantize_q4_0
    banks = [tuple(quant((rng.standard_normal(sh) * 0.1).astype(np.float32)) for sh in ((I, H), (I, H), (H, I)))
             for _ in range(E)]
    x = rng.standard_normal((T, H)).astype(np.float32)
    logits = rng.standard_normal((T, E))
    logits[1, [1, 4]] = logits[1, 2]  # a tie at the top: lower ids first
    res = oracle.moe_layer(x, qt, lambda e: banks[e], k, logits=logits)
    deq = [tuple(oracle.dequant(qt, b) for b in bank) for bank in banks]
    for t in range(T):
        chosen = sorted(range(E), key=lambda e: (-float(np.float32(logits[t, e])), e))[:k]
        assert res["ids"][t].tolist() == chosen
        z = [math.exp(logits[t, e] - logits[t, chosen[0]]) for e in chosen]
        want = np.zeros(H)
        for j, e in enumerate(chosen):
            y = _dense_ffn_loops(x[t].astype(np.float64), *deq[e])
            np.testing.assert_allclose(res["y_pairs"][t * k + j], y, rtol=1e-12, atol=1e-13)
            want = want + (z[j] / math.fsum(z)) * y
        np.testing.assert_allclose(res["out"][t], want, rtol=1e-12, atol=1e-13)


def test_quantize_act_q8_hand_blocks():
    """int8 block activations worked by hand: s = max|x| / 127, codes round
    half away from zero, an all-zero block has s = 0 and codes 0."""
    x = np.zeros(96, dtype=np.float32)
    x[0:6] = [0.5, -0.5, 1.5, 2.4999, -127.0, 127.0]   # s = 1
    x[32:36] = [63.5, 0.25, -0.25, 0.74]                # s = 0.5: 127, 1 (0.5 away), -1, 1 (1.48)
    q, s = oracle.quantize_act_q8(x)
    assert s.tolist() == [1.0, 0.5, 0.0]
    assert q[0:6].tolist() == [1, -1, 2, 2, -127, 127]
    assert q[32:36].tolist() == [127, 1, -1, 1]
    assert (q[64:] == 0).all()
    rng = np.random.default_rng(5)
    v = rng.standard_normal((4, 256)).astype(np.float32) * 3
    q, s = oracle.quantize_act_q8(v)
    assert np.abs(q).max() <= 127 and (np.abs(q).reshape(4, 8, 32).max(axis=2) == 127).all()
    err = np.abs(q.reshape(4, 8, 32) * s[..., None].astype(np.float64) - v.reshape(4, 8, 32))
    assert (err <= 0.5 * s[..., None] * (1 + 1e-6)).all()


@pytest.mark.parametrize("qt", ["q8_0", "q4_0"])
def test_matvec_q8a_exact_on_representable_activations(qt):
    """Activations that are integers with a +-127 in every block quantise
    exactly (s = 1), so the int8-activation product equals the plain product
    with the dequantised weights."""
    rng = np.random.default_rng(7)
    quant = gi.quantize_q8_0 if qt == "q8_0" else gi.quantize_q4_0
    blocks = quant((rng.standard_normal((40, 128)) * 0.05).astype(np.float32))
    x = rng.integers(-126, 127, 128).astype(np.float32)
    x[::32] = 127.0
    x[5::32] = -127.0
    xq, xs = oracle.quantize_act_q8(x)
    assert (xs == 1).all() and (xq == x).all()
    codes, d = oracle.block_codes_scales(qt, blocks)
    got = oracle.matvec_q8a(codes, d, xq, xs)
    np.testing.assert_allclose(got, oracle.dequant(qt, blocks) @ x.astype(np.float64), rtol=1e-13, atol=1e-13)


def test_expert_ffn_q8a_loops_and_closeness():
    """The int8-activation FFN equals the same steps written as plain loops
    on a tiny expert, and stays within 2e-2 (max relative) of the float FFN."""
    rng = np.random.default_rng(9)
    H, I = 64, 96
    banks = [gi.quantize_q4_0((rng.standard_normal(sh) * 0.1).astype(np.float32)) for sh in ((I, H), (I, H), (H, I))]
    x = rng.standard_normal((2, H)).astype(np.float32)
    got = oracle.expert_ffn_q8a(x, "q4_0", *banks)
    deq = [oracle.dequant("q4_0", b) for b in banks]

    def qrow(v):
        v = np.asarray(v, dtype=np.float32)
        out_q, out_s = [], []
        for b0 in range(0, len(v), 32):
            blk = v[b0:b0 + 32]
            s = np.float32(np.abs(blk).max() / np.float32(127))
            for val in blk:
                r = float(np.float32(val / s)) if s != 0 else 0.0
                out_q.append(0 if s == 0 else int(math.copysign(math.floor(abs(r) + 0.5), r)))
            out_s.append(float(s))
        return out_q, out_s

    def mv(bk, vq, vs):
        codes, d = oracle.block_codes_scales("q4_0", bk)
        return [math.fsum(float(d[r, b]) * vs[b] * sum(int(codes[r, b, j]) * vq[32 * b + j] for j in range(32))
                          for b in range(codes.shape[1])) for r in range(codes.shape[0])]

    for t in range(2):
        xq, xs = qrow(x[t])
        g, u = mv(banks[0], xq, xs), mv(banks[1], xq, xs)
        h = [gi_ / (1 + math.exp(-gi_)) * ui for gi_, ui in zip(g, u)]
        hq, hs = qrow(h)
        np.testing.assert_allclose(got[t], mv(banks[2], hq, hs), rtol=1e-12, atol=1e-12)
    ref = oracle.expert_ffn(x, *deq)
    assert np.abs(got - ref).max() / np.abs(ref).max() <= 2e-2


def test_combine_one_hot_is_gather():
    rng = np.random.default_rng(31)
    T, k, H = 5, 3, 4  # T != k so a transposed index fails
    y = rng.standard_normal((T * k, H))
    w = np.zeros((T, k))
    pick = rng.integers(0, k, T)
    w[np.arange(T), pick] = 1.0
    out = oracle.combine(y, w)
    np.testing.assert_array_equal(out, y[np.arange(T) * k + pick])
    w2 = rng.random((T, k))
    want = np.stack([sum(w2[t, j] * y[t * k + j] for j in range(k)) for t in range(T)])
    np.testing.assert_allclose(oracle.combine(y, w2), want, rtol=1e-15)


def test_layer_permutation_invariance_of_expert_labels():
    """Relabelling experts (permuting router rows and banks) leaves out unchanged."""
    rng = np.random.default_rng(37)
    H, I, E, k, T = 32, 64, 6, 2, 5
    banks = [tuple(gi.quantize_q8_0((rng.standard_normal(s) * 0.05).astype(np.float32))
                   for s in ((I, H), (I, H), (H, I))) for _ in range(E)]
    wr = rng.standard_normal((E, H)).astype(np.float32)
    x = rng.standard_normal((T, H)).astype(np.float32)
    a = oracle.moe_layer(x, "q8_0", lambda e: banks[e], k, router_w=wr)
    perm = rng.permutation(E)
    b = oracle.moe_layer(x, "q8_0", lambda e: banks[perm[e]], k, router_w=wr[perm])
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- LRU
def _ordered_dict_lru(trace, capacity):
    cache = collections.OrderedDict()
    hits = np.zeros(trace.shape, dtype=bool)
    for s in range(trace.shape[0]):
        for l in range(trace.shape[1]):
            protect = set()
            for j in range(trace.shape[2]):
                key = (l, int(trace[s, l, j]))
                if key in cache:
                    hits[s, l, j] = True
                    cache.move_to_end(key)
                else:
                    if len(cache) >= capacity:
                        for victim in cache:  # oldest first
                            if victim not in protect:
                                break
                        del cache[victim]
                    cache[key] = True
                protect.add(key)
    return hits


def test_lru_hand_trace():
    # capacity 3, one layer, two lookups per step
    trace = np.array([[[0, 1]], [[2, 0]], [[3, 1]], [[0, 2]]], dtype=np.int32)
    hit, ev = oracle.lru_simulate(trace, 3)
    assert hit.reshape(-1).tolist() == [False, False, False, True, False, False, True, False]
    # step 2: 3 evicts key 1 (LRU), then 1 evicts 2; step 3: 0 hit, 2 evicts 3
    assert [e[2] for e in ev] == [(0, 1), (0, 2), (0, 3)]


def test_lru_matches_ordered_dict_simulation():
    wl = gi.workload(5)
    trace = gi.cache_trace(wl, steps=96)
    for cap in (8, 20, 100, 816):
        hit, _ = oracle.lru_simulate(trace, cap)
        np.testing.assert_array_equal(hit, _ordered_dict_lru(trace, cap))


def test_lru_resize_hand_trace():
    # capacity 3, one layer, two lookups per step; shrink to 2 before step 2,
    # grow to 3 before step 3 (worked out by hand)
    trace = np.array([[[0, 1]], [[2, 3]], [[1, 3]], [[2, 1]]], dtype=np.int32)
    hit, ev = oracle.lru_simulate(trace, 3, resizes={(2, 0): 2, (3, 0): 3})
    # step 1: 3 evicts 0 (LRU).  Resize: {1, 2, 3} keeps the two most recent,
    # 2 and 3.  Step 2: 1 evicts 2 (3 was used later), 3 hits.  Step 3: room
    # for 2 again, 1 hits.
    assert hit.reshape(-1).tolist() == [False, False, False, False, False, True, False, True]
    assert ev == [(1, 0, (0, 0)), (2, 0, (0, 1)), (2, 0, (0, 2))]


def test_lru_resize_invariants():
    wl = gi.workload(5)
    trace = gi.cache_trace(wl, steps=48)
    base, _ = oracle.lru_simulate(trace, 100)
    # resizing to the current capacity changes nothing
    same, _ = oracle.lru_simulate(trace, 100, resizes={(10, 3): 100, (30, 0): 100})
    np.testing.assert_array_equal(same, base)
    # growing evicts nothing at the resize, and afterwards only misses of
    # keys never seen, or seen but evicted before the resize, can occur
    grown, ev = oracle.lru_simulate(trace, 40, resizes={(20, 0): 2048})
    assert all(s < 20 for s, _l, _k in ev)
    seen = set()
    for st in range(trace.shape[0]):
        for l in range(trace.shape[1]):
            for j in range(trace.shape[2]):
                key = (l, int(trace[st, l, j]))
                if st >= 20 and key in seen and key not in {e[2] for e in ev}:
                    assert grown[st, l, j]
                seen.add(key)
    # shrinking keeps the most recently used keys: after a shrink to the
    # lookups of one step, the next step's repeats still hit
    small, _ = oracle.lru_simulate(trace, 400, resizes={(24, 0): trace.shape[1] * trace.shape[2]})
    np.testing.assert_array_equal(small[:24], oracle.lru_simulate(trace[:24], 400)[0])


def test_lru_host_misses_hand_trace():
    # capacity 2, one layer: s0 [0, 1] copied; s1 [2, 0] with 2 on the host:
    # 2 misses and changes nothing, 0 hits; s2 [2, 1]: 2 now copied evicts
    # the LRU key 1 (0 was used at s1), then 1 misses and evicts 0.
    trace = np.array([[[0, 1]], [[2, 0]], [[2, 1]]], dtype=np.int32)
    hit, ev = oracle.lru_simulate(trace, 2, host={(1, 0): {2}})
    assert hit.reshape(-1).tolist() == [False, False, False, True, False, False]
    assert ev == [(2, 0, (0, 1)), (2, 0, (0, 0))]
    # without the host decision, 2 is inserted at s1 (evicting 0, so 0
    # misses too) and hits at s2
    hit2, _ = oracle.lru_simulate(trace, 2)
    assert hit2.reshape(-1).tolist() == [False, False, False, False, True, False]


def test_lru_host_invariants():
    wl = gi.workload(5)
    trace = gi.cache_trace(wl, steps=32)
    base, ev0 = oracle.lru_simulate(trace, 100)
    same, ev1 = oracle.lru_simulate(trace, 100, host={})
    np.testing.assert_array_equal(same, base)
    assert ev0 == ev1
    # every miss on the host: the cache never fills, so nothing ever hits
    everything = {(s, l): set(range(wl.E)) for s in range(trace.shape[0]) for l in range(trace.shape[1])}
    none_hit, ev = oracle.lru_simulate(trace, 100, host=everything)
    assert not none_hit.any() and ev == []
    # a resident expert cannot be sent to the host
    with pytest.raises(ValueError):
        oracle.lru_simulate(np.array([[[0]], [[0]]], dtype=np.int32), 2, host={(1, 0): {0}})


def test_lru_protects_current_layer_keys():
    trace = np.array([[[0, 1, 2]], [[3, 4, 5]]], dtype=np.int32)
    hit, ev = oracle.lru_simulate(trace, 3)
    assert not hit.any()
    assert [e[2] for e in ev] == [(0, 0), (0, 1), (0, 2)]
    with pytest.raises(ValueError):
        oracle.lru_simulate(trace, 2)
