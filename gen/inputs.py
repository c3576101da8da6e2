"""Seeded synthetic inputs for the five MoE-layer workloads.

Every tensor is drawn from its own NumPy PCG64 substream,
``SeedSequence(0, spawn_key=(workload, kind, a, b))``, so any single expert
of any layer can be regenerated on its own and in parallel.  Nothing here
computes the layer: the only arithmetic is the *quantiser* that turns fp32
draws into ggml Q8_0 / Q4_0 blocks (the weight format the pages name for
expert banks, "FreeToken" GitHub README, sections "Quant types" and "Known
limits") and the bias / trace recipes that describe the workloads.

Block formats (ggml array-of-structs, little endian), one block per 32
consecutive weights along the input dimension of a weight row:

* Q8_0: fp16 scale ``d`` (2 B) then 32 x int8 ``q``  -> 34 B.
  Quantiser: ``d = max|w| / 127``; ``q = round_half_away(w / d)``.
* Q4_0: fp16 scale ``d`` (2 B) then 16 B of nibbles  -> 18 B.  Byte ``j``
  holds element ``j`` in its low nibble and element ``j + 16`` in its high
  nibble.  Quantiser: ``m`` = signed element of largest magnitude (first on
  ties), ``d = m / -8``, ``q = min(15, floor(w / d + 8.5))``.
* Q4_1: fp16 ``d``, fp16 ``m`` then 16 B of nibbles (as Q4_0) -> 20 B;
  ``w = d q + m``.  Quantiser: ``m = min``, ``d = (max - min) / 15``,
  ``q = min(15, floor((w - m) / d + 0.5))``.
* Q5_0: fp16 ``d``, 4 B of fifth bits (bit ``j`` of the little-endian word
  for element ``j``), 16 B of nibbles -> 22 B; ``w = d (q - 16)``.
  Quantiser as Q4_0 with 16 for 8 and 31 for 15.
* Q5_1: fp16 ``d``, fp16 ``m``, 4 B of fifth bits, 16 B of nibbles -> 24 B;
  ``w = d q + m``.  Quantiser as Q4_1 with 31 for 15.

The quantisers only make input bytes; both the GPU library and the oracle
decode the same bytes.

Matrix orientation: every weight matrix is ``[out_rows][in_cols / 32]``
blocks; per expert the tensors are gate ``[I][H]``, up ``[I][H]`` and
down ``[H][I]``.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "QK", "BLOCK_BYTES", "KIND", "Workload", "WORKLOADS", "workload",
    "rng_for", "quantize_q8_0", "quantize_q4_0", "quantize_q4_1", "quantize_q5_0",
    "quantize_q5_1", "expert_weights_f32",
    "expert_blocks", "router_weight", "router_bias", "activations",
    "given_logits", "slot_permutation", "zipf_cdf", "cache_trace",
    "cache_trace_logits", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "generate_blocks_parallel", "weights_per_expert", "bytes_per_expert",
]

QK = 32
BLOCK_BYTES = {"q8_0": 34, "q4_0": 18, "q4_1": 20, "q5_0": 22, "q5_1": 24,
               "q4_k": 18, "q5_k": 22}  # bytes per 32 weights (Q4_K: 144, Q5_K: 176 per super-block of 256)

# substream "kind" field
KIND = {
    "x": 1, "router": 2, "gate": 3, "up": 4, "down": 5, "logits": 6,
    "slots": 7, "trace": 8, "trace_logits": 9,
}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes, weight format and routing source."""
    index: int            # substream id (1..5)
    name: str
    H: int                # hidden size
    E: int                # routed experts per layer
    k: int                # experts per token
    I: int                # expert FFN intermediate size
    qtype: str            # "q8_0" | "q4_0"
    batches: Tuple[int, ...]  # token counts T
    layers: int = 1
    x_dtype: str = "f32"  # "f32" | "bf16"
    router: str = "matrix"  # "matrix" | "logits" | "trace"
    zipf_bias_s: Optional[float] = None  # router bias -s*ln(e+1)
    cache_fraction: Optional[float] = None
    steps: Optional[int] = None
    trace_keep_p: Optional[float] = None
    trace_zipf_s: Optional[float] = None


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload(1, "tiny_q8_0", H=256, E=8, k=2, I=512, qtype="q8_0",
                 batches=(4,)),
        Workload(2, "decode_q8_0_h2048_e128", H=2048, E=128, k=8, I=768,
                 qtype="q8_0", batches=(1, 4, 16), layers=48),
        Workload(3, "prefill_q4_0_h2048_e128", H=2048, E=128, k=8, I=768,
                 qtype="q4_0", batches=(4096,), x_dtype="bf16",
                 router="logits"),
        Workload(4, "wide_q4_0_h2048_e512", H=2048, E=512, k=10, I=512,
                 qtype="q4_0", batches=(1, 64), zipf_bias_s=1.1),
        Workload(5, "cache_q4_0_h4096_e256", H=4096, E=256, k=8, I=2048,
                 qtype="q4_0", batches=(1,), layers=8, router="trace",
                 cache_fraction=0.4, steps=2048, trace_keep_p=0.7,
                 trace_zipf_s=1.0),
    ]
}


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        for w in WORKLOADS.values():
            if w.index == name_or_index:
                return w
        raise KeyError(name_or_index)
    return WORKLOADS[name_or_index]


def weights_per_expert(wl: Workload) -> int:
    return 3 * wl.H * wl.I


def bytes_per_expert(wl: Workload) -> int:
    return weights_per_expert(wl) // QK * BLOCK_BYTES[wl.qtype]


def rng_for(wl_index: int, kind: str, a: int = 0, b: int = 0) -> np.random.Generator:
    """Independent PCG64 stream for (workload, tensor kind, a, b), root seed 0."""
    ss = np.random.SeedSequence(0, spawn_key=(wl_index, KIND[kind], a, b))
    return np.random.Generator(np.random.PCG64(ss))


# --------------------------------------------------------------------------
# bf16 helpers (NumPy has no bf16 dtype: bf16 travels as uint16 bit patterns)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# quantisers (input preparation only)
# --------------------------------------------------------------------------
def _round_half_away(x32: np.ndarray) -> np.ndarray:
    x = x32.astype(np.float64)
    return np.trunc(x + np.copysign(0.5, x))


def quantize_q8_0(w: np.ndarray) -> np.ndarray:
    """fp32 [rows, K] -> uint8 [rows, K/32, 34] ggml Q8_0 blocks."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    assert K % QK == 0
    b = w.reshape(rows, K // QK, QK)
    amax = np.abs(b).max(axis=2)
    d = (amax / np.float32(127.0)).astype(np.float32)
    nz = d != 0
    inv = np.zeros_like(d)
    inv[nz] = np.float32(1.0) / d[nz]
    q = _round_half_away(b * inv[..., None]).astype(np.int8)
    out = np.empty((rows, K // QK, 34), dtype=np.uint8)
    out[..., 0:2] = d.astype(np.float16).view(np.uint8).reshape(rows, K // QK, 2)
    out[..., 2:] = q.view(np.uint8)
    return out


def quantize_q4_0(w: np.ndarray) -> np.ndarray:
    """fp32 [rows, K] -> uint8 [rows, K/32, 18] ggml Q4_0 blocks."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    assert K % QK == 0
    b = w.reshape(rows, K // QK, QK)
    idx = np.abs(b).argmax(axis=2)  # first occurrence on ties
    m = np.take_along_axis(b, idx[..., None], axis=2)[..., 0]
    d = (m / np.float32(-8.0)).astype(np.float32)
    nz = d != 0
    inv = np.zeros_like(d)
    inv[nz] = np.float32(1.0) / d[nz]
    t = (b * inv[..., None] + np.float32(8.5)).astype(np.float32)
    q = np.minimum(np.trunc(t), 15).astype(np.uint8)
    out = np.empty((rows, K // QK, 18), dtype=np.uint8)
    out[..., 0:2] = d.astype(np.float16).view(np.uint8).reshape(rows, K // QK, 2)
    out[..., 2:] = q[..., :16] | (q[..., 16:] << 4)
    return out


def _fp16_bytes(v: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(v.astype(np.float16)).view(np.uint8).reshape(*v.shape, 2)


def _pack_nibbles(q: np.ndarray) -> np.ndarray:
    """codes [..., 32] (0..15 after masking) -> 16 bytes: j low, j + 16 high."""
    q = q.astype(np.uint8) & 0x0F
    return q[..., :16] | (q[..., 16:] << 4)


def _pack_fifth_bits(q: np.ndarray) -> np.ndarray:
    """codes [..., 32] in 0..31 -> 4 bytes: bit j of the little-endian word is bit 4 of code j."""
    bits = (q.astype(np.uint32) >> 4) & 1
    word = (bits << np.arange(32, dtype=np.uint32)).sum(axis=-1, dtype=np.uint64).astype("<u4")
    return np.ascontiguousarray(word).view(np.uint8).reshape(*q.shape[:-1], 4)


def _affine_codes(b: np.ndarray, top: int):
    """min / max quantiser: m = min, d = (max - min) / top, q = min(top, floor((w - m) / d + 0.5))."""
    mn = b.min(axis=2)
    d = ((b.max(axis=2) - mn) / np.float32(top)).astype(np.float32)
    nz = d != 0
    inv = np.zeros_like(d)
    inv[nz] = np.float32(1.0) / d[nz]
    t = ((b - mn[..., None]) * inv[..., None] + np.float32(0.5)).astype(np.float32)
    q = np.minimum(np.trunc(t), top).astype(np.uint8)
    return d, mn, q


def quantize_q4_1(w: np.ndarray) -> np.ndarray:
    """fp32 [rows, K] -> uint8 [rows, K/32, 20] ggml Q4_1 blocks."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    d, mn, q = _affine_codes(w.reshape(rows, K // QK, QK), 15)
    out = np.empty((rows, K // QK, 20), dtype=np.uint8)
    out[..., 0:2] = _fp16_bytes(d)
    out[..., 2:4] = _fp16_bytes(mn)
    out[..., 4:] = _pack_nibbles(q)
    return out


def quantize_q5_0(w: np.ndarray) -> np.ndarray:
    """fp32 [rows, K] -> uint8 [rows, K/32, 22] ggml Q5_0 blocks."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    b = w.reshape(rows, K // QK, QK)
    idx = np.abs(b).argmax(axis=2)
    m = np.take_along_axis(b, idx[..., None], axis=2)[..., 0]
    d = (m / np.float32(-16.0)).astype(np.float32)
    nz = d != 0
    inv = np.zeros_like(d)
    inv[nz] = np.float32(1.0) / d[nz]
    t = (b * inv[..., None] + np.float32(16.5)).astype(np.float32)
    q = np.minimum(np.trunc(t), 31).astype(np.uint8)
    out = np.empty((rows, K // QK, 22), dtype=np.uint8)
    out[..., 0:2] = _fp16_bytes(d)
    out[..., 2:6] = _pack_fifth_bits(q)
    out[..., 6:] = _pack_nibbles(q)
    return out


def quantize_q5_1(w: np.ndarray) -> np.ndarray:
    """fp32 [rows, K] -> uint8 [rows, K/32, 24] ggml Q5_1 blocks."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    d, mn, q = _affine_codes(w.reshape(rows, K // QK, QK), 31)
    out = np.empty((rows, K // QK, 24), dtype=np.uint8)
    out[..., 0:2] = _fp16_bytes(d)
    out[..., 2:4] = _fp16_bytes(mn)
    out[..., 4:8] = _pack_fifth_bits(q)
    out[..., 8:] = _pack_nibbles(q)
    return out


def _round_half_away_f32(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    return np.where(v >= 0, np.floor(v + 0.5), np.ceil(v - 0.5))


def pack_q4_k(d: np.ndarray, dmin: np.ndarray, sc: np.ndarray, mn: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Q4_K super-blocks from their fields: d, dmin fp32 [...] (stored as
    fp16), 6-bit scales and mins [..., 8], codes [..., 8, 32] in 0..15 ->
    uint8 [..., 144]: d, dmin, 12 bytes of packed scales and mins, 128 bytes
    of nibbles (sub-block 2i low and 2i+1 high in bytes 32i .. 32i+31)."""
    sc = np.asarray(sc).astype(np.uint8)
    mn = np.asarray(mn).astype(np.uint8)
    q = np.asarray(q).astype(np.uint8)
    out = np.empty(sc.shape[:-1] + (144,), dtype=np.uint8)
    out[..., 0:2] = _fp16_bytes(np.asarray(d, dtype=np.float32))
    out[..., 2:4] = _fp16_bytes(np.asarray(dmin, dtype=np.float32))
    for j in range(4):
        out[..., 4 + j] = (sc[..., j] & 63) | ((sc[..., j + 4] >> 4) << 6)
        out[..., 8 + j] = (mn[..., j] & 63) | ((mn[..., j + 4] >> 4) << 6)
        out[..., 12 + j] = (sc[..., j + 4] & 0x0F) | ((mn[..., j + 4] & 0x0F) << 4)
    for i in range(4):
        out[..., 16 + 32 * i:48 + 32 * i] = (q[..., 2 * i, :] & 0x0F) | ((q[..., 2 * i + 1, :] & 0x0F) << 4)
    return out


def pack_q5_k(d: np.ndarray, dmin: np.ndarray, sc: np.ndarray, mn: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Q5_K super-blocks from their fields (as pack_q4_k, codes in 0..31)
    -> uint8 [..., 176]: d, dmin, the 12 scale bytes, 32 bytes qh (bit j of
    byte l = bit 4 of element l of sub-block j), 128 bytes of low nibbles
    laid out as in Q4_K."""
    q = np.asarray(q).astype(np.uint8)
    k4 = pack_q4_k(d, dmin, sc, mn, q & 0x0F)
    out = np.empty(k4.shape[:-1] + (176,), dtype=np.uint8)
    out[..., 0:16] = k4[..., 0:16]
    hi = (q >> 4) & 1  # [..., 8, 32]
    qh = np.zeros(q.shape[:-2] + (32,), dtype=np.uint8)
    for j in range(8):
        qh |= (hi[..., j, :] << j).astype(np.uint8)
    out[..., 16:48] = qh
    out[..., 48:176] = k4[..., 16:144]
    return out


def _quantize_k(w: np.ndarray, top: int):
    """Fields of K-quant super-blocks with weight codes in 0..top."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    sb = w.reshape(rows, K // 256, 8, 32)
    off = np.maximum(-sb.min(axis=3), np.float32(0)).astype(np.float32)
    step = ((sb.max(axis=3) + off) / np.float32(top)).astype(np.float32)
    d = (step.max(axis=2) / np.float32(63)).astype(np.float16).astype(np.float32)
    dmin = (off.max(axis=2) / np.float32(63)).astype(np.float16).astype(np.float32)

    def codes(v, s, top):
        out = np.zeros(v.shape, dtype=np.float64)
        nz = np.broadcast_to(s != 0, v.shape)
        ratio = np.zeros(v.shape, dtype=np.float32)
        ratio[nz] = (np.broadcast_to(v, v.shape)[nz] / np.broadcast_to(s, v.shape)[nz]).astype(np.float32)
        out[nz] = _round_half_away_f32(ratio[nz])
        return np.clip(out, 0, top).astype(np.uint8)

    sc = codes(step, d[..., None], 63)
    mn = codes(off, dmin[..., None], 63)
    eff_d = (d[..., None] * sc.astype(np.float32)).astype(np.float32)
    eff_m = (dmin[..., None] * mn.astype(np.float32)).astype(np.float32)
    q = codes((sb + eff_m[..., None]).astype(np.float32), eff_d[..., None], top)
    return d, dmin, sc, mn, q


def quantize_q4_k(w: np.ndarray) -> np.ndarray:
    """fp32 [rows, K] -> uint8 [rows, K/256, 144] ggml Q4_K super-blocks.

    Harness quantiser (both sides read the same bytes): per sub-block of 32
    the offset m = max(0, -min) and the step s = (max + m) / 15; per
    super-block d = max step / 63 and dmin = max offset / 63, stored as fp16;
    6-bit scale and min codes round(s / d), round(m / dmin); weight codes
    round((w + dmin * min) / (d * scale)) clamped to 0..15 (rounding half away
    from zero, in fp32)."""
    return pack_q4_k(*_quantize_k(w, 15))


def quantize_q5_k(w: np.ndarray) -> np.ndarray:
    """fp32 [rows, K] -> uint8 [rows, K/256, 176] ggml Q5_K super-blocks:
    quantize_q4_k's recipe with steps (max + m) / 31 and codes in 0..31."""
    return pack_q5_k(*_quantize_k(w, 31))


_QUANT = {"q8_0": quantize_q8_0, "q4_0": quantize_q4_0, "q4_1": quantize_q4_1, "q5_0": quantize_q5_0,
          "q5_1": quantize_q5_1, "q4_k": quantize_q4_k, "q5_k": quantize_q5_k}


# --------------------------------------------------------------------------
# weights, router, activations
# --------------------------------------------------------------------------
def expert_weights_f32(wl: Workload, layer: int, expert: int):
    """fp32 N(0, 0.02) draws (gate [I,H], up [I,H], down [H,I]) before quantisation."""
    sigma = np.float32(0.02)
    out = []
    for kind, shape in (("gate", (wl.I, wl.H)), ("up", (wl.I, wl.H)), ("down", (wl.H, wl.I))):
        g = rng_for(wl.index, kind, layer, expert)
        out.append(g.standard_normal(shape, dtype=np.float32) * sigma)
    return tuple(out)


def expert_blocks(wl: Workload, layer: int, expert: int):
    """ggml blocks (gate, up, down) of one expert: uint8 [rows, cols/32, bpb]."""
    q = _QUANT[wl.qtype]
    return tuple(q(m) for m in expert_weights_f32(wl, layer, expert))


def generate_blocks_parallel(wl: Workload, pairs: Sequence[Tuple[int, int]],
                             consume, threads: Optional[int] = None) -> None:
    """Generate expert_blocks for many (layer, expert) pairs on a thread pool.

    ``consume(layer, expert, (gate, up, down))`` is called from the worker
    threads; NumPy releases the GIL inside the heavy loops.
    """
    threads = threads or min(16, os.cpu_count() or 1)

    def job(le):
        l, e = le
        consume(l, e, expert_blocks(wl, l, e))

    with ThreadPoolExecutor(threads) as ex:
        for _ in ex.map(job, pairs):
            pass


def router_weight(wl: Workload, layer: int = 0) -> np.ndarray:
    """Router matrix Wr [E, H] fp32, N(0, 0.02) (row e maps hidden -> logit e)."""
    g = rng_for(wl.index, "router", layer)
    return g.standard_normal((wl.E, wl.H), dtype=np.float32) * np.float32(0.02)


def router_bias(wl: Workload) -> Optional[np.ndarray]:
    """Zipf-shaped logit bias b[e] = -s * ln(e + 1) (expert e has rank e + 1)."""
    if wl.zipf_bias_s is None:
        return None
    e = np.arange(wl.E, dtype=np.float64)
    return (-wl.zipf_bias_s * np.log(e + 1.0)).astype(np.float32)


def activations(wl: Workload, T: int, step: int = 0) -> np.ndarray:
    """Token activations [T, H] N(0, 1): fp32, or bf16 bit patterns (uint16)."""
    g = rng_for(wl.index, "x", T, step)
    x = g.standard_normal((T, wl.H), dtype=np.float32)
    if wl.x_dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def given_logits(wl: Workload, T: int, layer: int = 0) -> np.ndarray:
    """Router logits supplied directly: i.i.d. N(0, 1) fp32 [T, E], one
    independent draw per layer."""
    g = rng_for(wl.index, "logits", T, layer)
    return g.standard_normal((T, wl.E), dtype=np.float32)


def slot_permutation(wl: Workload, layer: int = 0, n_slots: Optional[int] = None) -> np.ndarray:
    """Seeded expert -> VRAM slot map (int32 [E]) for fully resident pools."""
    g = rng_for(wl.index, "slots", layer)
    n = n_slots or wl.E
    return g.permutation(n)[: wl.E].astype(np.int32)


# --------------------------------------------------------------------------
# expert-cache routing trace
# --------------------------------------------------------------------------
def zipf_cdf(n: int, s: float) -> np.ndarray:
    r = np.arange(1, n + 1, dtype=np.float64)
    p = r ** (-s)
    c = np.cumsum(p)
    return c / c[-1]


def cache_trace(wl: Workload, steps: Optional[int] = None) -> np.ndarray:
    """Expert ids int32 [steps, layers, k] with temporal locality.

    Per layer, independently: step 0 takes k distinct Zipf(s) draws over
    ranks 1..E (rank r is expert r-1, repeats rejected).  Each later step
    keeps every id of the previous step with probability p (in order), then
    fills up with Zipf draws, rejecting ids already chosen.
    """
    steps = steps or wl.steps
    L, E, k = wl.layers, wl.E, wl.k
    cdf = zipf_cdf(E, wl.trace_zipf_s)
    out = np.empty((steps, L, k), dtype=np.int32)
    for l in range(L):
        g = rng_for(wl.index, "trace", l)
        prev: List[int] = []
        for s in range(steps):
            if s == 0:
                chosen: List[int] = []
            else:
                keep = g.random(len(prev)) < wl.trace_keep_p
                chosen = [e for e, kp in zip(prev, keep) if kp]
            while len(chosen) < k:
                e = int(np.searchsorted(cdf, g.random(), side="right"))
                e = min(e, E - 1)
                if e not in chosen:
                    chosen.append(e)
            out[s, l] = chosen
            prev = chosen
    return out


def cache_trace_logits(wl: Workload, trace: np.ndarray, step: int) -> np.ndarray:
    """Router logits [layers, E] fp32 for one step of the trace.

    The step's chosen ids get i.i.d. N(0, 1) logits; every other expert gets
    -1e4, so a top-k selection picks exactly the chosen set.
    """
    L, E = wl.layers, wl.E
    out = np.full((L, E), -1.0e4, dtype=np.float32)
    for l in range(L):
        g = rng_for(wl.index, "trace_logits", l, step)
        out[l, trace[step, l]] = g.standard_normal(trace.shape[2], dtype=np.float32)
    return out
