"""CPU oracle for the routed-expert MoE layer forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it, and it shares no code with the GPU library: it reads the logical
ggml block bytes produced by ``gen`` and computes everything in float64 with
plain NumPy steps that can be checked against the definitions by eye.

Sources.  The pages describe FreeToken, an engine that keeps the full expert
pool in host memory and uses VRAM as an expert cache
("FreeToken github moe: Setup Guide & MoE Runtime Comparison", introduction;
"FreeToken Inference Engine: 3x Speed Boost for MoE Models", section "From
Static Allocation to Dynamic Scheduling").  The expert banks are ggml
blocks of the standard types (Q4_0, Q4_1, Q5_0, Q5_1, Q8_0) and the
Q4_K K-quant held in one slot pool of one type (FreeToken fork README, sections "Quant types" and
"Known limits").  Each token activates only a
subset of the experts (setup guide, introduction).  The steps below are the
plainest reading of that layer: softmax over expert logits, keep the k
largest (ties to the lower expert id), renormalise the kept probabilities,
group token/expert pairs by expert, run a SwiGLU expert FFN per pair, and
sum the FFN outputs weighted by the renormalised probabilities.

Decision precision.  Top-k selection is an integer decision taken on fp32
logits, the precision the GPU kernel decides in: ``topk_select`` casts its
input to float32 before ordering.  Everything else is float64.

NaN logits.  The pages do not mention them.  Here a NaN logit reads as
-inf in every routing step (selection, softmax, top-k gap): it is never
chosen over a number, ties with -inf (lower id first), and has
probability 0.

Parity pins.  Every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, brute force or independent simulations.  The full
layer output at large sizes has no external values to compare against; it is
pinned only through its pinned parts ("parity unpinned" beyond them).
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

QK = 32  # weights per block, every format here


# --------------------------------------------------------------------------
# 1. block dequantisation (ggml Q8_0 / Q4_0 / Q4_1 / Q5_0 / Q5_1 and Q4_K;
#    FreeToken fork README, "Quant types": the standard and K-quant rows)
# --------------------------------------------------------------------------
def _block_scale(blocks: np.ndarray) -> np.ndarray:
    """fp16 little-endian scale in bytes 0..1 of every block, as float64."""
    return np.ascontiguousarray(blocks[..., 0:2]).view(np.float16)[..., 0].astype(np.float64)


def dequant_q8_0(blocks: np.ndarray) -> np.ndarray:
    """uint8 [..., nblk, 34] -> float64 [..., nblk*32]; w_i = d * q_i (q int8)."""
    d = _block_scale(blocks)
    q = np.ascontiguousarray(blocks[..., 2:34]).view(np.int8).astype(np.float64)
    w = d[..., None] * q
    return w.reshape(*blocks.shape[:-2], blocks.shape[-2] * QK)


def dequant_q4_0(blocks: np.ndarray) -> np.ndarray:
    """uint8 [..., nblk, 18] -> float64 [..., nblk*32]; w = d * (q - 8).

    Byte j of the 16 nibble bytes carries element j (low nibble) and
    element j + 16 (high nibble).
    """
    d = _block_scale(blocks)
    nib = blocks[..., 2:18]
    q = np.concatenate([nib & 0x0F, nib >> 4], axis=-1).astype(np.float64)
    w = d[..., None] * (q - 8.0)
    return w.reshape(*blocks.shape[:-2], blocks.shape[-2] * QK)


def _half(blocks: np.ndarray, at: int) -> np.ndarray:
    """fp16 little-endian in bytes at..at+1 of every block, as float64."""
    return np.ascontiguousarray(blocks[..., at:at + 2]).view(np.float16)[..., 0].astype(np.float64)


def _nibbles(qs: np.ndarray) -> np.ndarray:
    """16 bytes -> 32 codes: element j in the low nibble of byte j, element
    j + 16 in its high nibble."""
    return np.concatenate([qs & 0x0F, qs >> 4], axis=-1).astype(np.int64)


def _high_bits(qh: np.ndarray) -> np.ndarray:
    """4 bytes read as a little-endian uint32 -> 32 bits, bit j for element j."""
    word = np.ascontiguousarray(qh).view("<u4")[..., 0].astype(np.int64)
    return (word[..., None] >> np.arange(32)) & 1


def dequant_q4_1(blocks: np.ndarray) -> np.ndarray:
    """uint8 [..., nblk, 20] -> float64; d (fp16), m (fp16), 16 nibble bytes:
    w = d * q + m with q in 0..15."""
    d, m = _half(blocks, 0), _half(blocks, 2)
    q = _nibbles(blocks[..., 4:20]).astype(np.float64)
    w = d[..., None] * q + m[..., None]
    return w.reshape(*blocks.shape[:-2], blocks.shape[-2] * QK)


def dequant_q5_0(blocks: np.ndarray) -> np.ndarray:
    """uint8 [..., nblk, 22] -> float64; d (fp16), 4 bytes of fifth bits,
    16 nibble bytes: q = nibble + 16 * bit in 0..31, w = d * (q - 16)."""
    d = _half(blocks, 0)
    q = _nibbles(blocks[..., 6:22]) + 16 * _high_bits(blocks[..., 2:6])
    w = d[..., None] * (q.astype(np.float64) - 16.0)
    return w.reshape(*blocks.shape[:-2], blocks.shape[-2] * QK)


def dequant_q5_1(blocks: np.ndarray) -> np.ndarray:
    """uint8 [..., nblk, 24] -> float64; d, m (fp16), 4 bytes of fifth bits,
    16 nibble bytes: q = nibble + 16 * bit in 0..31, w = d * q + m."""
    d, m = _half(blocks, 0), _half(blocks, 2)
    q = _nibbles(blocks[..., 8:24]) + 16 * _high_bits(blocks[..., 4:8])
    w = d[..., None] * q.astype(np.float64) + m[..., None]
    return w.reshape(*blocks.shape[:-2], blocks.shape[-2] * QK)


QK_K = 256  # weights per K-quant super-block


def q4_k_scales_mins(sc12: np.ndarray):
    """The 12 packed bytes of a Q4_K super-block -> (scales, mins), int64
    [..., 8], each a 6-bit field of sub-block j = 0..7.  Sub-blocks 0-3:
    the low six bits of byte j (scale) and of byte j + 4 (min).  Sub-blocks
    4-7: byte j + 4 gives the low four bits (scale in its low nibble, min
    in its high nibble), and the top two bits of byte j - 4 (scale) and of
    byte j (min) give bits 4-5."""
    b = np.asarray(sc12).astype(np.int64)
    sc = np.empty(b.shape[:-1] + (8,), dtype=np.int64)
    mn = np.empty(b.shape[:-1] + (8,), dtype=np.int64)
    for j in range(4):
        sc[..., j] = b[..., j] & 63
        mn[..., j] = b[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (b[..., j + 4] & 0x0F) | ((b[..., j - 4] >> 6) << 4)
        mn[..., j] = (b[..., j + 4] >> 4) | ((b[..., j] >> 6) << 4)
    return sc, mn


def dequant_q4_k(blocks: np.ndarray) -> np.ndarray:
    """uint8 [..., nsb, 144] -> float64 [..., nsb*256] (ggml Q4_K, a K-quant
    of the FreeToken fork README's "Quant types" table).  A super-block of
    256 weights: fp16 d, fp16 dmin, 12 bytes of 6-bit scales and mins of its
    8 sub-blocks of 32, then 128 bytes of nibbles.  Bytes 32i .. 32i+31 hold
    sub-block 2i in their low nibbles and sub-block 2i+1 in their high
    nibbles, element l of either sub-block in byte 32i + l.  Weight l of
    sub-block j: d * scale_j * q - dmin * min_j."""
    d, dmin = _half(blocks, 0), _half(blocks, 2)
    sc, mn = q4_k_scales_mins(blocks[..., 4:16])
    qs = blocks[..., 16:144].astype(np.int64)
    q = np.empty(blocks.shape[:-1] + (8, 32), dtype=np.int64)
    for i in range(4):
        chunk = qs[..., 32 * i:32 * i + 32]
        q[..., 2 * i, :] = chunk & 0x0F
        q[..., 2 * i + 1, :] = chunk >> 4
    w = (d[..., None, None] * sc[..., None]) * q - (dmin[..., None] * mn)[..., None]
    return w.reshape(*blocks.shape[:-2], blocks.shape[-2] * QK_K)


def dequant_q5_k(blocks: np.ndarray) -> np.ndarray:
    """uint8 [..., nsb, 176] -> float64 [..., nsb*256] (ggml Q5_K, the
    five-bit K-quant of the same "Quant types" table).  Q4_K's super-block
    with 32 bytes qh between the scale bytes and the nibbles: fp16 d, fp16
    dmin, 12 scale bytes, qh, 128 nibble bytes.  Code q of element l of
    sub-block j = its nibble (as in Q4_K) + 16 * bit j of qh byte l, in
    0..31; weight = d * scale_j * q - dmin * min_j."""
    d, dmin = _half(blocks, 0), _half(blocks, 2)
    sc, mn = q4_k_scales_mins(blocks[..., 4:16])
    qh = blocks[..., 16:48].astype(np.int64)
    qs = blocks[..., 48:176].astype(np.int64)
    q = np.empty(blocks.shape[:-1] + (8, 32), dtype=np.int64)
    for j in range(8):
        chunk = qs[..., 32 * (j // 2):32 * (j // 2) + 32]
        nib = chunk >> 4 if j % 2 else chunk & 0x0F
        q[..., j, :] = nib + 16 * ((qh >> j) & 1)
    w = (d[..., None, None] * sc[..., None]) * q - (dmin[..., None] * mn)[..., None]
    return w.reshape(*blocks.shape[:-2], blocks.shape[-2] * QK_K)


_DEQUANT = {"q8_0": dequant_q8_0, "q4_0": dequant_q4_0, "q4_1": dequant_q4_1, "q5_0": dequant_q5_0,
            "q5_1": dequant_q5_1, "q4_k": dequant_q4_k, "q5_k": dequant_q5_k}


def dequant(qtype: str, blocks: np.ndarray) -> np.ndarray:
    if qtype not in _DEQUANT:
        raise ValueError(f"unsupported block type {qtype!r}")
    return _DEQUANT[qtype](blocks)


# --------------------------------------------------------------------------
# 2-5. router: logits, softmax, top-k, renormalisation
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, router_w: np.ndarray,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * Wr[e, h] (+ b[e]); Wr is [E, H]."""
    l = np.asarray(x, dtype=np.float64) @ np.asarray(router_w, dtype=np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def nan_as_minus_inf(l: np.ndarray) -> np.ndarray:
    """A NaN logit reads as -inf: it is never chosen over a number and its
    probability is 0.  The pages say nothing about NaN router logits; this
    is the reading under which every routing step stays defined (a NaN
    would otherwise poison the softmax of the whole row)."""
    l = np.asarray(l)
    return np.where(np.isnan(l), -np.inf, l).astype(l.dtype)


def softmax(l: np.ndarray) -> np.ndarray:
    """Row softmax, max-shifted for range; NaN logits count as -inf."""
    l = nan_as_minus_inf(np.asarray(l, dtype=np.float64))
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def topk_select(l: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest fp32 logits per row, ordered (logit desc, id asc).

    Selecting on logits equals selecting on their softmax (a monotone map)
    and avoids false ties where exp() rounds two logits to one value.  NaN
    counts as -inf (so it ties with -inf and loses to every number).
    """
    l32 = nan_as_minus_inf(np.asarray(l, dtype=np.float32))
    order = np.argsort(-l32, axis=-1, kind="stable")  # equal keys keep id order
    return order[..., :k].astype(np.int32)


def renormalize(p: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w[t, j] = p[t, ids[t, j]] / sum_j' p[t, ids[t, j']]."""
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=-1)
    return sel / sel.sum(axis=-1, keepdims=True)


def route(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """softmax -> top-k -> renormalise.  Returns (ids int32 [T,k], w float64 [T,k])."""
    ids = topk_select(logits, k)
    w = renormalize(softmax(logits), ids)
    return ids, w


def topk_gap(l: np.ndarray, k: int) -> np.ndarray:
    """Per row: k-th largest minus (k+1)-th largest logit (inf when k == E).

    NaN counts as -inf; two equal values (two -inf included) have gap 0.
    """
    s = -np.sort(-nan_as_minus_inf(np.asarray(l, dtype=np.float64)), axis=-1)
    if k >= s.shape[-1]:
        return np.full(s.shape[:-1], np.inf)
    a, b = s[..., k - 1], s[..., k]
    with np.errstate(invalid="ignore"):
        return np.where(a == b, 0.0, a - b)


# --------------------------------------------------------------------------
# 6. permutation: group pairs p = t*k + j by expert (stable)
# --------------------------------------------------------------------------
def permute(ids: np.ndarray, E: int):
    """Stable counting sort of pairs by expert id.

    Returns (offsets [E+1], sorted_pairs [P], pair_pos [P], active ids).
    ``sorted_pairs[offsets[e]:offsets[e+1]]`` lists the pairs routed to
    expert e in ascending pair order; ``pair_pos`` is the inverse map;
    ``active`` lists the experts with at least one pair, ascending.
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    P = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    sorted_pairs = np.empty(P, dtype=np.int64)
    pair_pos = np.empty(P, dtype=np.int64)
    for p in range(P):
        e = flat[p]
        sorted_pairs[cursor[e]] = p
        pair_pos[p] = cursor[e]
        cursor[e] += 1
    active = np.array([e for e in range(E) if counts[e] > 0], dtype=np.int64)
    return (offsets.astype(np.int32), sorted_pairs.astype(np.int32),
            pair_pos.astype(np.int32), active.astype(np.int32))


# --------------------------------------------------------------------------
# 7. expert FFN (SwiGLU) and 8. combine
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_ffn(x_rows: np.ndarray, wg: np.ndarray, wu: np.ndarray,
               wd: np.ndarray) -> np.ndarray:
    """SwiGLU FFN of one expert on rows x [n, H]: Wd (silu(Wg x) * (Wu x)).

    wg, wu: [I, H]; wd: [H, I] (float64 dequantised weights).
    """
    x = np.asarray(x_rows, dtype=np.float64)
    g = x @ wg.T
    u = x @ wu.T
    return (silu(g) * u) @ wd.T


def moe_ffn_pairs(x: np.ndarray, ids: np.ndarray, E: int, qtype: str,
                  get_blocks, act_q8: bool = False) -> np.ndarray:
    """y_pairs [T*k, H]: FFN output of every pair p = t*k + j in pair order.

    ``get_blocks(e)`` returns the ggml blocks (gate, up, down) of expert e.
    ``act_q8``: the int8-activation FFN (expert_ffn_q8a) instead.
    """
    T, k = ids.shape
    x32 = np.asarray(x, dtype=np.float32)
    x = np.asarray(x, dtype=np.float64)
    offsets, sorted_pairs, _, active = permute(ids, E)
    y = np.zeros((T * k, x.shape[1]), dtype=np.float64)
    for e in active:
        pairs = sorted_pairs[offsets[e]:offsets[e + 1]]
        gb, ub, db = get_blocks(int(e))
        if act_q8:
            y[pairs] = expert_ffn_q8a(x32[pairs // k], qtype, gb, ub, db)
            continue
        wg, wu, wd = dequant(qtype, gb), dequant(qtype, ub), dequant(qtype, db)
        y[pairs] = expert_ffn(x[pairs // k], wg, wu, wd)
    return y


# --------------------------------------------------------------------------
# 7b. decode with int8 activations: the fork README's W4A8 scheme
#     ("DeepSeek-V4-Flash" section: 4-bit weights against 8-bit activations
#     in the decode kernels, not bit-comparable with an fp32 reference)
# --------------------------------------------------------------------------
def quantize_act_q8(x: np.ndarray):
    """fp32 [..., K] -> (codes int64 [..., K] in -127..127, scales fp32
    [..., K/32]).  Per block of 32: s = max |x| / 127 and the code x / s
    rounded half away from zero, both divisions in fp32; s = 0 gives codes
    0.  (The pages give no formula; this is the plainest symmetric int8
    block quantiser.)"""
    x32 = np.asarray(x, dtype=np.float32)
    b = x32.reshape(*x32.shape[:-1], -1, QK)
    s = (np.abs(b).max(axis=-1) / np.float32(127)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1), s)
    ratio = (b / safe[..., None]).astype(np.float32).astype(np.float64)
    q = np.where(ratio >= 0, np.floor(ratio + 0.5), np.ceil(ratio - 0.5))
    q = np.where((s == 0)[..., None], 0.0, np.clip(q, -127, 127)).astype(np.int64)
    return q.reshape(x32.shape), s


def block_codes_scales(qtype: str, blocks: np.ndarray):
    """(signed codes int64 [..., nblk, 32], scales float64 [..., nblk]) of
    the types whose weight is d * code: Q8_0 (code q) and Q4_0 (code q - 8)."""
    d = _block_scale(blocks)
    if qtype == "q8_0":
        codes = np.ascontiguousarray(blocks[..., 2:34]).view(np.int8).astype(np.int64)
    elif qtype == "q4_0":
        nib = blocks[..., 2:18]
        codes = np.concatenate([nib & 0x0F, nib >> 4], axis=-1).astype(np.int64) - 8
    else:
        raise ValueError(f"int8-activation decode takes Q8_0 and Q4_0 banks, not {qtype!r}")
    return codes, d


def matvec_q8a(codes: np.ndarray, d: np.ndarray, aq: np.ndarray, a_s: np.ndarray) -> np.ndarray:
    """rows [R, nblk, 32] codes with scales [R, nblk] against one quantised
    activation row (codes [nblk*32], scales [nblk]):
    y_r = sum_b d[r, b] * a_s[b] * (sum_j codes[r, b, j] * aq[b, j]),
    the inner sums exact integers."""
    inner = (codes * aq.reshape(1, -1, QK)).sum(axis=-1)
    return (d * a_s.astype(np.float64)[None, :] * inner).sum(axis=-1)


def expert_ffn_q8a(x_rows: np.ndarray, qtype: str, gate_blocks, up_blocks, down_blocks) -> np.ndarray:
    """SwiGLU FFN of one expert with int8 block activations: x quantised,
    g and u by matvec_q8a, h = silu(g) u, h rounded to fp32 (the precision
    the h rows are kept in) and quantised, y by matvec_q8a."""
    gc, gd = block_codes_scales(qtype, gate_blocks)
    uc, ud = block_codes_scales(qtype, up_blocks)
    dc, dd = block_codes_scales(qtype, down_blocks)
    out = []
    for x in np.asarray(x_rows, dtype=np.float32):
        xq, xs = quantize_act_q8(x)
        g, u = matvec_q8a(gc, gd, xq, xs), matvec_q8a(uc, ud, xq, xs)
        hq, hs = quantize_act_q8((silu(g) * u).astype(np.float32))
        out.append(matvec_q8a(dc, dd, hq, hs))
    return np.array(out).reshape(-1, dc.shape[0])


def combine(y_pairs: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t] = sum over j ascending of w[t, j] * y[t*k + j]."""
    T, k = w.shape
    y = np.asarray(y_pairs, dtype=np.float64).reshape(T, k, -1)
    out = np.zeros((T, y.shape[2]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y[:, j, :]
    return out


def moe_layer(x: np.ndarray, qtype: str, get_blocks, k: int, *,
              router_w: Optional[np.ndarray] = None,
              bias: Optional[np.ndarray] = None,
              logits: Optional[np.ndarray] = None,
              act_q8: bool = False) -> Dict[str, np.ndarray]:
    """Whole layer: route -> permute -> expert FFN -> combine.

    Router logits are computed from x and Wr, or taken as given.  Returns
    a dict with logits, ids, w, y_pairs, out and the top-k logit gap.
    ``act_q8``: the expert FFN with int8 block activations.
    """
    if logits is None:
        logits = router_logits(x, router_w, bias)
    logits = np.asarray(logits, dtype=np.float64)
    ids, w = route(logits, k)
    y = moe_ffn_pairs(x, ids, logits.shape[1], qtype, get_blocks, act_q8=act_q8)
    return {"logits": logits, "ids": ids, "w": w, "y_pairs": y,
            "out": combine(y, w), "gap": topk_gap(logits, k)}


# --------------------------------------------------------------------------
# 9. expert cache: global LRU over (layer, expert) keys
#    (FreeToken fork README, "About": global LRU expert caching; setup guide:
#    a shared LRU follows token-level routing locality; 3x-speed article,
#    "From Static Allocation to Dynamic Scheduling": VRAM is a cache over the
#    host-resident pool and only missing experts move over PCIe)
# --------------------------------------------------------------------------
def lru_simulate(trace: np.ndarray, capacity: int, resizes: Optional[Dict[Tuple[int, int], int]] = None,
                 host: Optional[Dict[Tuple[int, int], set]] = None):
    """Replay lookups in order; returns (hit bool [steps, L, n], evicted keys).

    For every step, every layer and every id of that (step, layer) in
    order, the key (layer, id) is looked up.  A resident key is a hit and
    becomes most recently used.  A missing key is inserted; when the cache
    is full the least recently used key is evicted first, never one looked
    up earlier in the same (step, layer).  The cache starts empty.

    resizes {(step, layer): capacity}: the cache size changes at run time
    ("FreeToken Inference Engine: 3x Speed Boost for MoE Models", section
    "Dynamic Cache Adjustment Experiments"), just before that (step,
    layer)'s lookups; the most recently used keys stay, up to the new
    capacity, and the others are evicted.

    host {(step, layer): ids}: missing experts of that (step, layer) that
    are computed on the CPU instead of being moved to the GPU ("FreeToken
    Inference Engine: 3x Speed Boost for MoE Models", section "Q* Strategy:
    Intelligently Choosing Where to Compute").  Their lookups are misses
    that leave the cache as it was: nothing is inserted, refreshed or
    evicted for them.
    """
    steps, L, n = trace.shape
    host = host or {}
    last_use: Dict[Tuple[int, int], int] = {}
    clock = 0
    hit = np.zeros(trace.shape, dtype=bool)
    evicted: List[Tuple[int, int, Tuple[int, int]]] = []
    resizes = resizes or {}
    for s in range(steps):
        for l in range(L):
            if (s, l) in resizes:
                capacity = resizes[(s, l)]
                while len(last_use) > capacity:
                    victim = min(last_use, key=lambda kk: last_use[kk])
                    del last_use[victim]
                    evicted.append((s, l, victim))
            current = set()
            on_host = host.get((s, l), ())
            for j in range(n):
                key = (l, int(trace[s, l, j]))
                if key[1] in on_host:
                    if key in last_use:
                        raise ValueError(f"expert {key} is resident, so it cannot be computed on the host")
                    continue
                clock += 1
                if key in last_use:
                    hit[s, l, j] = True
                else:
                    if len(last_use) >= capacity:
                        candidates = [kk for kk in last_use if kk not in current]
                        if not candidates:
                            raise ValueError("cache capacity below the keys of one layer")
                        victim = min(candidates, key=lambda kk: last_use[kk])
                        del last_use[victim]
                        evicted.append((s, l, victim))
                last_use[key] = clock
                current.add(key)
    return hit, evicted
