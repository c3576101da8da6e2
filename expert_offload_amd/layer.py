"""Run one MoE layer forward through libmoe's entry points.

``LayerBuffers`` owns the device buffers of one batch size; ``forward``
issues moe_route -> moe_permute -> moe_expert_ffn -> moe_combine on one
stream.  ``pack_expert`` / ``SlotPool`` move ggml blocks (host) into the
device slot layout (libmoe's packer) and into a device slot pool.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _lib as L


def pack_expert(qtype: str, H: int, I: int, gate, up, down) -> np.ndarray:
    """ggml blocks (host) -> one slot in the device layout (host uint8)."""
    q = L.QTYPE[qtype]
    out = np.empty(L.moe_slot_bytes(q, H, I), dtype=np.uint8)
    L.moe_pack_expert(q, H, I, np.ascontiguousarray(gate), np.ascontiguousarray(up),
                      np.ascontiguousarray(down), out)
    return out


class SlotPool:
    """A device slot pool of ``n_slots`` experts of one block type."""

    def __init__(self, qtype: str, H: int, I: int, n_slots: int, device="cuda"):
        self.qtype, self.H, self.I, self.n_slots = qtype, H, I, n_slots
        self.q = L.QTYPE[qtype]
        self.slot_bytes = L.moe_slot_bytes(self.q, H, I)
        self.data = torch.empty(n_slots * self.slot_bytes, dtype=torch.uint8, device=device)

    def base(self, first_slot: int = 0) -> int:
        return self.data.data_ptr() + first_slot * self.slot_bytes

    def put(self, slot: int, packed: np.ndarray) -> None:
        dst = self.data[slot * self.slot_bytes:(slot + 1) * self.slot_bytes]
        dst.copy_(torch.from_numpy(packed))


class LayerBuffers:
    """Device buffers for one layer forward over T tokens."""

    def __init__(self, T: int, H: int, I: int, E: int, k: int, qtype: str, device="cuda",
                 mode: int = L.MODE_DECODE, x_dtype: int = L.DTYPE_F32):
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.q = L.QTYPE[qtype]
        self.mode, self.x_dtype = mode, x_dtype
        P = max(T * k, 1)
        i32, f32 = torch.int32, torch.float32
        self.logits = torch.empty((max(T, 1), E), dtype=f32, device=device)
        self.ids = torch.empty((max(T, 1), k), dtype=i32, device=device)
        self.w = torch.empty((max(T, 1), k), dtype=f32, device=device)
        self.offsets = torch.empty(E + 1, dtype=i32, device=device)
        self.sorted_pairs = torch.empty(P, dtype=i32, device=device)
        self.pair_pos = torch.empty(P, dtype=i32, device=device)
        self.active = torch.empty(E + 1, dtype=i32, device=device)
        self.y = torch.empty((P, H), dtype=f32, device=device)
        self.out = torch.empty((max(T, 1), H), dtype=f32, device=device)
        probe = L.moe_ffn_args(qtype=self.q, H=H, I=I, T=T, k=k, E=E, mode=mode, x_dtype=x_dtype, n_slots=1,
                               slot_bytes=L.moe_slot_bytes(self.q, H, I))
        self.ws_bytes = L.moe_expert_ffn_workspace_size(probe)
        # workspaces start zeroed; the library leaves their counters zero
        self.ws = torch.zeros(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.route_ws = torch.zeros(max(L.moe_route_permute_workspace_size(T, k, E), 256),
                                    dtype=torch.uint8, device=device)
        self.perm_ws = torch.zeros(max(L.moe_permute_workspace_size(T, k, E), 256), dtype=torch.uint8,
                                   device=device)


def forward(ctx: L.Ctx, buf: LayerBuffers, pool_base: int, slot_bytes: int, n_slots: int, slot_table, x,
            router_w=None, bias=None, logits_in=None, expert_mask=None, stream=None,
            steps=("route", "permute", "ffn", "combine"), fused: bool = False) -> torch.Tensor:
    """One layer forward; returns ``buf.out`` (valid in stream order).

    ``fused``: True = moe_route_permute, then moe_expert_ffn with the
    combine folded in (two calls); "layer" = moe_decode_layer (one call);
    "static" = moe_decode_layer_static (one call, no workspace); otherwise
    the four entry points one after another.
    """
    T, H, I, E, k = buf.T, buf.H, buf.I, buf.E, buf.k
    if fused == "layer":
        args = L.make_ffn_args(pool_base, slot_bytes, n_slots, buf.q, H, I, T, k, E, slot_table, x,
                               buf.offsets, buf.sorted_pairs, buf.active, buf.y, buf.mode,
                               ws=buf.ws, ws_bytes=buf.ws.numel(), x_dtype=buf.x_dtype,
                               topk_w=buf.w, out=buf.out)
        L.moe_decode_layer(ctx, args, router_w, bias, logits_in, buf.logits, buf.ids, buf.pair_pos, stream=stream)
        return buf.out
    if fused == "static":  # moe_decode_layer_static: the library's own scratch, no workspace passed
        args = L.make_ffn_args(pool_base, slot_bytes, n_slots, buf.q, H, I, T, k, E, slot_table, x,
                               buf.offsets, buf.sorted_pairs, buf.active, buf.y, buf.mode,
                               ws=None, ws_bytes=0, x_dtype=buf.x_dtype, topk_w=buf.w, out=buf.out)
        L.moe_decode_layer_static(ctx, args, router_w, bias, logits_in, buf.logits, buf.ids, buf.pair_pos,
                                  stream=stream)
        return buf.out
    if fused and expert_mask is None:
        L.moe_route_permute(ctx, x, router_w, bias, logits_in, T, H, E, k, buf.logits, buf.ids, buf.w,
                            buf.offsets, buf.sorted_pairs, buf.pair_pos, buf.active, buf.route_ws,
                            buf.route_ws.numel(), stream=stream, x_dtype=buf.x_dtype)
        args = L.make_ffn_args(pool_base, slot_bytes, n_slots, buf.q, H, I, T, k, E, slot_table, x,
                               buf.offsets, buf.sorted_pairs, buf.active, buf.y, buf.mode,
                               ws=buf.ws, ws_bytes=buf.ws.numel(), x_dtype=buf.x_dtype,
                               topk_w=buf.w, out=buf.out)
        L.moe_expert_ffn(ctx, args, stream=stream)
        return buf.out
    if "route" in steps:
        L.moe_route(ctx, x, router_w, bias, logits_in, T, H, E, k, buf.logits, buf.ids, buf.w,
                    stream=stream, x_dtype=buf.x_dtype)
    if "permute" in steps:
        L.moe_permute(ctx, buf.ids, T, k, E, buf.offsets, buf.sorted_pairs, buf.pair_pos,
                      buf.active, buf.perm_ws, buf.perm_ws.numel(), stream=stream)
    if "ffn" in steps:
        args = L.make_ffn_args(pool_base, slot_bytes, n_slots, buf.q, H, I, T, k, E, slot_table, x,
                               buf.offsets, buf.sorted_pairs, buf.active, buf.y, buf.mode,
                               ws=buf.ws, ws_bytes=buf.ws.numel(), expert_mask=expert_mask,
                               x_dtype=buf.x_dtype)
        L.moe_expert_ffn(ctx, args, stream=stream)
    if "combine" in steps:
        L.moe_combine(ctx, buf.y, buf.w, T, k, H, buf.out, stream=stream)
    return buf.out


class CachedLayers:
    """Decode through L layers whose experts live in a pinned host pool,
    with a VRAM expert cache (cache_slot_table_* / prefetch_expert).

    Per layer: route on the GPU; the ids come back to the host (the host
    cannot know them earlier, since a layer's routing depends on that
    layer's input); the host looks them up in the global LRU; the FFN runs
    on the hits while the misses are copied on a side stream; then the FFN
    runs on the misses and the combine forms the output.
    """

    def __init__(self, ctx: L.Ctx, qtype: str, H: int, I: int, E: int, k: int, L_layers: int,
                 n_slots: int, host_pool: torch.Tensor, device="cuda"):
        self.ctx, self.qtype, self.H, self.I, self.E, self.k, self.L = ctx, qtype, H, I, E, k, L_layers
        self.q = L.QTYPE[qtype]
        self.slot_bytes = L.moe_slot_bytes(self.q, H, I)
        self.n_slots = n_slots
        self.d_pool = torch.empty((n_slots + 2) * self.slot_bytes, dtype=torch.uint8, device=device)
        self.host_pool = host_pool
        self.cache = L.cache_slot_table_create(L_layers, E, n_slots, self.q, H, I, self.d_pool, host_pool)
        self.table = L.cache_slot_table_device(self.cache)
        self.copy_stream = torch.cuda.Stream()
        self.buf = LayerBuffers(1, H, I, E, k, qtype, device=device)
        self.ids_host = torch.empty((1, k), dtype=torch.int32, pin_memory=True)
        self.mask_host = torch.zeros((2, E), dtype=torch.int32, pin_memory=True)
        self.mask_dev = torch.zeros((2, E), dtype=torch.int32, device=device)
        self.ev_ids = torch.cuda.Event()
        self.misses_per_layer = []

    def layer(self, l: int, x: torch.Tensor, logits: torch.Tensor, stream=None, native: bool = True) -> torch.Tensor:
        """Layer `l` with given router logits; `native` runs the whole
        sequence in one library call (cache_decode_layer), otherwise step by
        step from Python (same calls, same results)."""
        b = self.buf
        s = stream or torch.cuda.current_stream()
        if native:
            before = self.stats()[1]
            L.cache_decode_layer(self.cache, self.ctx, l, x, None, None, logits, 1, self.k, b.logits, b.ids, b.w,
                                 b.offsets, b.sorted_pairs, b.pair_pos, b.active, b.y, b.ws, b.ws.numel(), b.out,
                                 self.copy_stream, s)
            self.misses_per_layer.append(self.stats()[1] - before)
            return b.out
        L.moe_route_permute(self.ctx, x, None, None, logits, 1, self.H, self.E, self.k, b.logits, b.ids, b.w,
                            b.offsets, b.sorted_pairs, b.pair_pos, b.active, None, 0, stream=s)
        self.ids_host.copy_(b.ids, non_blocking=True)
        self.ev_ids.record(s)
        self.ev_ids.synchronize()
        ids = self.ids_host.numpy()[0]
        slots, misses = L.cache_slot_table_lookup(self.cache, l, ids)
        self.misses_per_layer.append(len(misses))
        hit = np.isin(np.arange(self.E), ids) & ~np.isin(np.arange(self.E), misses)
        self.mask_host[0].copy_(torch.from_numpy(hit.astype(np.int32)))
        self.mask_host[1].copy_(torch.from_numpy(np.isin(np.arange(self.E), misses).astype(np.int32)))
        self.mask_dev.copy_(self.mask_host, non_blocking=True)
        table = self.table + 4 * l * self.E
        base = self.d_pool.data_ptr()
        common = dict(ws=b.ws, ws_bytes=b.ws.numel(), x_dtype=L.DTYPE_F32)
        if hit.any():
            args = L.make_ffn_args(base, self.slot_bytes, self.n_slots + 2, self.q, self.H, self.I, 1, self.k,
                                   self.E, table, x, b.offsets, b.sorted_pairs, b.active, b.y, L.MODE_DECODE,
                                   expert_mask=self.mask_dev[0], **common)
            L.moe_expert_ffn(self.ctx, args, stream=s)
        if len(misses):
            for e in misses:
                L.prefetch_expert(self.cache, l, int(e), self.copy_stream, s)
            args = L.make_ffn_args(base, self.slot_bytes, self.n_slots + 2, self.q, self.H, self.I, 1, self.k,
                                   self.E, table, x, b.offsets, b.sorted_pairs, b.active, b.y, L.MODE_DECODE,
                                   expert_mask=self.mask_dev[1], **common)
            L.moe_expert_ffn(self.ctx, args, stream=s)
        L.moe_combine(self.ctx, b.y, b.w, 1, self.k, self.H, b.out, stream=s)
        L.cache_mark_layer_done(self.cache, l, s)
        return b.out

    def resize(self, n_slots: int, in_place: bool = False, stream=None) -> None:
        """Change the cache capacity at run time.  By default the experts
        kept move into a new pool of exactly (n_slots + 2) slots and the old
        one is released; in_place keeps the current allocation (shrinking
        only)."""
        if in_place:
            if n_slots > self.n_slots:
                raise ValueError("an in-place resize can only shrink the cache")
            L.cache_slot_table_resize(self.cache, n_slots, None, stream)
        else:
            pool = torch.empty((n_slots + 2) * self.slot_bytes, dtype=torch.uint8, device=self.d_pool.device)
            L.cache_slot_table_resize(self.cache, n_slots, pool, stream)
            self.d_pool = pool
        self.n_slots = n_slots

    def set_miss_policy(self, policy: int, host_threads: int = 0) -> None:
        """L.MISS_COPY, L.MISS_HOST or L.MISS_QSTAR for the native layer path."""
        L.cache_set_miss_policy(self.cache, policy, host_threads)

    def last_misses(self):
        """(copied ids, host ids, number of host ids left out of the cache)
        of the last native layer call."""
        return L.cache_last_misses(self.cache)

    def miss_stats(self):
        return L.cache_miss_stats(self.cache)

    def stats(self):
        return L.cache_slot_table_stats(self.cache)

    def close(self):
        torch.cuda.synchronize()
        self.cache.close()


class StreamedPrefill:
    """Prefill through L layers whose experts live in a pinned host pool and
    stream through two device buffers of one layer each (prefill_stream_*):
    the next layer's experts are copied while the current layer computes."""

    def __init__(self, ctx: L.Ctx, qtype: str, H: int, I: int, E: int, k: int, L_layers: int, T_max: int,
                 host_pool: torch.Tensor, device="cuda"):
        self.ctx, self.qtype, self.H, self.I, self.E, self.k, self.L = ctx, qtype, H, I, E, k, L_layers
        self.q = L.QTYPE[qtype]
        self.slot_bytes = L.moe_slot_bytes(self.q, H, I)
        self.d_bufs = torch.empty(2 * E * self.slot_bytes, dtype=torch.uint8, device=device)
        self.host_pool = host_pool
        self.ps = L.prefill_stream_create(L_layers, E, self.q, H, I, self.d_bufs, host_pool)
        self.copy_stream = torch.cuda.Stream()
        self.buf = LayerBuffers(T_max, H, I, E, k, qtype, device=device, mode=L.MODE_PREFILL,
                                x_dtype=L.DTYPE_BF16)

    def layer(self, l: int, x: torch.Tensor, logits: torch.Tensor, out: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
        """Layer `l` over x (bf16 [T, H]) with given router logits (fp32
        [T, E]); writes `out` (fp32 [T, H], default the buffers' own)."""
        b = self.buf
        T = x.shape[0]
        out = b.out if out is None else out
        args = L.make_ffn_args(None, self.slot_bytes, self.E, self.q, self.H, self.I, T, self.k, self.E, None, x,
                               b.offsets, b.sorted_pairs, b.active, b.y, L.MODE_PREFILL, ws=b.ws,
                               ws_bytes=b.ws.numel(), x_dtype=L.DTYPE_BF16, topk_w=b.w, out=out)
        L.prefill_stream_layer(self.ps, self.ctx, l, args, None, None, logits, None, b.ids, b.pair_pos,
                               b.route_ws, b.route_ws.numel(), self.copy_stream, stream)
        return out

    def stats(self):
        return L.prefill_stream_stats(self.ps)

    def close(self):
        torch.cuda.synchronize()
        self.ps.close()
