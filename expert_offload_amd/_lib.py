"""ctypes binding of libmoe (include/moe.h): same entry-point names, argument
marshalling only.  Tensors are passed as their data pointers; PyTorch is
used for device memory and streams.  Every computation happens in libmoe.

PyTorch is imported before the library is loaded so that libmoe binds to
the HIP runtime PyTorch already loaded (one runtime, one device context).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch  # noqa: F401  (must precede loading libmoe)

# MOE_LIB_PATH selects another build of the library (the host-sanitizer
# build that the CPU tests load under AddressSanitizer)
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK = 0
ERRORS = {
    -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED_QTYPE", -3: "MOE_ERR_MIXED_QTYPE",
    -4: "MOE_ERR_ALIGNMENT", -5: "MOE_ERR_WORKSPACE", -6: "MOE_ERR_NOT_RESIDENT",
    -7: "MOE_ERR_NOT_PINNED", -8: "MOE_ERR_CAPACITY", -9: "MOE_ERR_HIP",
}
QTYPE = {"q4_0": 2, "q4_1": 3, "q5_0": 6, "q5_1": 7, "q8_0": 8, "q4_k": 12, "q5_k": 13}
DTYPE_F32, DTYPE_BF16 = 0, 1
MODE_DECODE, MODE_PREFILL, MODE_DECODE_Q8A = 0, 1, 2

# every symbol include/moe.h declares
EXPORTS = (
    "moe_last_error", "moe_ctx_create", "moe_ctx_destroy", "moe_ctx_check", "moe_qtype_info",
    "moe_slot_bytes", "moe_pack_expert", "moe_pack_matrix", "moe_route",
    "moe_permute_workspace_size", "moe_permute", "moe_expert_ffn_workspace_size",
    "moe_expert_ffn", "moe_combine", "moe_dequantize", "cache_slot_table_create",
    "cache_slot_table_lookup", "cache_slot_table_device", "cache_slot_table_stats",
    "cache_slot_table_destroy", "prefetch_expert", "cache_mark_layer_done", "cache_slot_table_resize",
    "moe_check_bank_types", "moe_ctx_set_timing", "moe_ctx_kernel_time",
    "moe_route_permute_workspace_size", "moe_route_permute", "moe_decode_layer", "cache_decode_layer",
    "prefill_stream_create", "prefill_stream_layer", "prefill_stream_stats", "prefill_stream_destroy",
    "moe_host_expert_ffn", "moe_host_has_avx512", "cache_set_miss_policy", "cache_miss_stats",
    "cache_last_misses", "moe_decode_layer_static", "moe_static_scratch_bytes",
)


class MoeError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn} -> {ERRORS.get(code, code)}: {msg}")
        self.code = code
        self.name = ERRORS.get(code, str(code))


class moe_ffn_args(ctypes.Structure):
    _fields_ = [
        ("pool_base", ctypes.c_void_p), ("slot_bytes", ctypes.c_size_t), ("n_slots", ctypes.c_int),
        ("qtype", ctypes.c_int),
        ("H", ctypes.c_int), ("I", ctypes.c_int), ("T", ctypes.c_int), ("k", ctypes.c_int),
        ("E", ctypes.c_int), ("slot_table", ctypes.c_void_p), ("x", ctypes.c_void_p),
        ("x_dtype", ctypes.c_int), ("expert_offsets", ctypes.c_void_p),
        ("sorted_pairs", ctypes.c_void_p), ("active", ctypes.c_void_p),
        ("expert_mask", ctypes.c_void_p), ("y_pairs", ctypes.c_void_p), ("mode", ctypes.c_int),
        ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
        ("topk_w", ctypes.c_void_p), ("out", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree); fails loudly when it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run expert_offload_amd.build.build() "
                          "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, sz, i32p, i64p = (ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t,
                             ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64))
    ip = ctypes.POINTER(ctypes.c_int)
    szp = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_ctx_create": (i, [i, ctypes.POINTER(vp)]),
        "moe_ctx_destroy": (i, [vp]),
        "moe_ctx_check": (i, [vp, vp]),
        "moe_qtype_info": (i, [i, ip, ip]),
        "moe_slot_bytes": (i, [i, i, i, szp]),
        "moe_pack_expert": (i, [i, i, i, vp, vp, vp, vp, sz]),
        "moe_pack_matrix": (i, [i, i, i, vp, vp, sz]),
        "moe_route": (i, [vp, vp, i, vp, vp, vp, i, i, i, i, vp, vp, vp, vp]),
        "moe_permute_workspace_size": (i, [i, i, i, szp]),
        "moe_permute": (i, [vp, vp, i, i, i, vp, vp, vp, vp, vp, sz, vp]),
        "moe_expert_ffn_workspace_size": (i, [ctypes.POINTER(moe_ffn_args), szp]),
        "moe_expert_ffn": (i, [vp, ctypes.POINTER(moe_ffn_args), vp]),
        "moe_decode_layer": (i, [vp, ctypes.POINTER(moe_ffn_args), vp, vp, vp, vp, vp, vp, vp]),
        "moe_decode_layer_static": (i, [vp, ctypes.POINTER(moe_ffn_args), vp, vp, vp, vp, vp, vp, vp]),
        "moe_static_scratch_bytes": (sz, []),
        "moe_combine": (i, [vp, vp, vp, i, i, i, vp, vp]),
        "moe_dequantize": (i, [vp, i, vp, i, i, i, vp, vp]),
        "cache_slot_table_create": (i, [i, i, i, i, i, i, vp, vp, ctypes.POINTER(vp)]),
        "cache_slot_table_lookup": (i, [vp, i, i32p, i, i32p, i32p, ip]),
        "cache_slot_table_device": (vp, [vp]),
        "cache_slot_table_stats": (i, [vp, i64p, i64p]),
        "cache_slot_table_destroy": (i, [vp]),
        "cache_slot_table_resize": (i, [vp, i, vp, vp]),
        "prefetch_expert": (i, [vp, i, i, vp, vp, i32p]),
        "cache_mark_layer_done": (i, [vp, i, vp]),
        "cache_set_miss_policy": (i, [vp, i, i]),
        "cache_miss_stats": (i, [vp, i64p, i64p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
        "cache_last_misses": (i, [vp, i32p, ip, i32p, ip, ip]),
        "moe_host_expert_ffn": (i, [i, i, i, vp, vp, i, vp, i, i]),
        "moe_host_has_avx512": (i, []),
        "prefill_stream_create": (i, [i, i, i, i, i, vp, vp, ctypes.POINTER(vp)]),
        "prefill_stream_layer": (i, [vp, vp, i, ctypes.POINTER(moe_ffn_args), vp, vp, vp, vp, vp, vp, vp, sz,
                                     vp, vp]),
        "prefill_stream_stats": (i, [vp, i64p, i64p]),
        "prefill_stream_destroy": (i, [vp]),
        "cache_decode_layer": (i, [vp, vp, i, vp, vp, vp, vp, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                   vp, vp]),
        "moe_check_bank_types": (i, [i, i, ip, ip]),
        "moe_ctx_set_timing": (i, [vp, i]),
        "moe_route_permute_workspace_size": (i, [i, i, i, szp]),
        "moe_route_permute": (i, [vp, vp, i, vp, vp, vp, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_ctx_kernel_time": (i, [vp, ctypes.c_char_p, ip, ctypes.POINTER(ctypes.c_double)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(rc: int, fn: str):
    if rc != MOE_OK:
        raise MoeError(rc, fn, lib().moe_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, torch.Tensor):
        if not t.is_contiguous():
            raise ValueError("libmoe takes contiguous tensors")
        return t.data_ptr()
    raise TypeError(f"expected a tensor, an int pointer or None, got {type(t)}")


def _dev_ptr(t) -> Optional[int]:
    if isinstance(t, torch.Tensor) and not t.is_cuda:
        raise ValueError("expected a device tensor")
    return _ptr(t)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ----------------------------------------------------------------- context
class Ctx:
    def __init__(self, device: int = 0):
        h = ctypes.c_void_p()
        _check(lib().moe_ctx_create(device, ctypes.byref(h)), "moe_ctx_create")
        self.handle = h
        self.device = device

    def close(self):
        if self.handle:
            lib().moe_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_ctx_create(device: int = 0) -> Ctx:
    return Ctx(device)


def moe_ctx_check(ctx: Ctx, stream=None) -> None:
    _check(lib().moe_ctx_check(ctx.handle, _stream(stream)), "moe_ctx_check")


def moe_ctx_set_timing(ctx: Ctx, enable: bool) -> None:
    _check(lib().moe_ctx_set_timing(ctx.handle, int(bool(enable))), "moe_ctx_set_timing")


def moe_ctx_kernel_time(ctx: Ctx, kernel: str) -> Tuple[int, float]:
    """(number of timed launches, summed milliseconds) of one kernel."""
    n, ms = ctypes.c_int(), ctypes.c_double()
    _check(lib().moe_ctx_kernel_time(ctx.handle, kernel.encode(), ctypes.byref(n), ctypes.byref(ms)),
           "moe_ctx_kernel_time")
    return n.value, ms.value


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_qtype_info(qtype: int) -> Tuple[int, int]:
    a, b = ctypes.c_int(), ctypes.c_int()
    _check(lib().moe_qtype_info(qtype, ctypes.byref(a), ctypes.byref(b)), "moe_qtype_info")
    return a.value, b.value


def moe_slot_bytes(qtype: int, H: int, I: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_slot_bytes(qtype, H, I, ctypes.byref(n)), "moe_slot_bytes")
    return n.value


def moe_pack_expert(qtype: int, H: int, I: int, gate, up, down, dst) -> None:
    """Host numpy/torch CPU buffers: ggml blocks -> device slot layout in dst."""
    def hp(a):
        if isinstance(a, torch.Tensor):
            return _ptr(a)
        return a.ctypes.data
    nbytes = dst.nbytes if hasattr(dst, "nbytes") else dst.numel() * dst.element_size()
    _check(lib().moe_pack_expert(qtype, H, I, hp(gate), hp(up), hp(down), hp(dst), nbytes),
           "moe_pack_expert")


def moe_pack_matrix(qtype: int, rows: int, cols: int, blocks, dst) -> None:
    _check(lib().moe_pack_matrix(qtype, rows, cols, blocks.ctypes.data, dst.ctypes.data, dst.nbytes),
           "moe_pack_matrix")


def moe_check_bank_types(qtypes) -> int:
    import numpy as np
    q = np.ascontiguousarray(qtypes, dtype=np.int32)
    out = ctypes.c_int()
    _check(lib().moe_check_bank_types(q.shape[0], q.shape[1],
                                      q.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
                                      ctypes.byref(out)), "moe_check_bank_types")
    return out.value


# ----------------------------------------------------------------- compute
def moe_route(ctx: Ctx, x, router_w, bias, logits_in, T: int, H: int, E: int, k: int,
              logits_out, topk_ids, topk_w, stream=None, x_dtype: Optional[int] = None) -> None:
    if x_dtype is None:
        x_dtype = DTYPE_BF16 if (isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16) else DTYPE_F32
    _check(lib().moe_route(ctx.handle, _dev_ptr(x), x_dtype, _dev_ptr(router_w), _dev_ptr(bias),
                           _dev_ptr(logits_in), T, H, E, k, _dev_ptr(logits_out), _dev_ptr(topk_ids),
                           _dev_ptr(topk_w), _stream(stream)), "moe_route")


def moe_route_permute_workspace_size(T: int, k: int, E: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_route_permute_workspace_size(T, k, E, ctypes.byref(n)),
           "moe_route_permute_workspace_size")
    return n.value


def moe_route_permute(ctx: Ctx, x, router_w, bias, logits_in, T: int, H: int, E: int, k: int,
                      logits_out, topk_ids, topk_w, expert_offsets, sorted_pairs, pair_pos, active,
                      ws, ws_bytes: int, stream=None, x_dtype: Optional[int] = None) -> None:
    if x_dtype is None:
        x_dtype = DTYPE_BF16 if (isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16) else DTYPE_F32
    _check(lib().moe_route_permute(ctx.handle, _dev_ptr(x), x_dtype, _dev_ptr(router_w), _dev_ptr(bias),
                                   _dev_ptr(logits_in), T, H, E, k, _dev_ptr(logits_out),
                                   _dev_ptr(topk_ids), _dev_ptr(topk_w), _dev_ptr(expert_offsets),
                                   _dev_ptr(sorted_pairs), _dev_ptr(pair_pos), _dev_ptr(active),
                                   _dev_ptr(ws), ws_bytes, _stream(stream)), "moe_route_permute")


def moe_permute_workspace_size(T: int, k: int, E: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_permute_workspace_size(T, k, E, ctypes.byref(n)), "moe_permute_workspace_size")
    return n.value


def moe_permute(ctx: Ctx, topk_ids, T: int, k: int, E: int, expert_offsets, sorted_pairs, pair_pos,
                active, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(lib().moe_permute(ctx.handle, _dev_ptr(topk_ids), T, k, E, _dev_ptr(expert_offsets),
                             _dev_ptr(sorted_pairs), _dev_ptr(pair_pos), _dev_ptr(active),
                             _dev_ptr(ws), ws_bytes, _stream(stream)), "moe_permute")


def make_ffn_args(pool, slot_bytes, n_slots, qtype, H, I, T, k, E, slot_table, x, expert_offsets,
                  sorted_pairs, active, y_pairs, mode, ws=None, ws_bytes=0, expert_mask=None,
                  x_dtype=None, topk_w=None, out=None) -> moe_ffn_args:
    if x_dtype is None:
        x_dtype = DTYPE_BF16 if (isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16) else DTYPE_F32
    return moe_ffn_args(
        pool_base=_dev_ptr(pool), slot_bytes=slot_bytes, n_slots=n_slots, qtype=qtype, H=H, I=I, T=T, k=k, E=E,
        slot_table=_dev_ptr(slot_table), x=_dev_ptr(x), x_dtype=x_dtype,
        expert_offsets=_dev_ptr(expert_offsets), sorted_pairs=_dev_ptr(sorted_pairs),
        active=_dev_ptr(active), expert_mask=_dev_ptr(expert_mask), y_pairs=_dev_ptr(y_pairs),
        mode=mode, ws=_dev_ptr(ws), ws_bytes=ws_bytes, topk_w=_dev_ptr(topk_w), out=_dev_ptr(out))


def moe_expert_ffn_workspace_size(args: moe_ffn_args) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_expert_ffn_workspace_size(ctypes.byref(args), ctypes.byref(n)),
           "moe_expert_ffn_workspace_size")
    return n.value


def moe_expert_ffn(ctx: Ctx, args: moe_ffn_args, stream=None) -> None:
    _check(lib().moe_expert_ffn(ctx.handle, ctypes.byref(args), _stream(stream)), "moe_expert_ffn")


def moe_decode_layer(ctx: Ctx, args: moe_ffn_args, router_w, bias, logits_in, logits_out, topk_ids, pair_pos,
                     stream=None) -> None:
    _check(lib().moe_decode_layer(ctx.handle, ctypes.byref(args), _dev_ptr(router_w), _dev_ptr(bias),
                                  _dev_ptr(logits_in), _dev_ptr(logits_out), _dev_ptr(topk_ids),
                                  _dev_ptr(pair_pos), _stream(stream)), "moe_decode_layer")


def moe_decode_layer_static(ctx: Ctx, args: moe_ffn_args, router_w, bias, logits_in, logits_out, topk_ids,
                            pair_pos, stream=None) -> None:
    _check(lib().moe_decode_layer_static(ctx.handle, ctypes.byref(args), _dev_ptr(router_w), _dev_ptr(bias),
                                         _dev_ptr(logits_in), _dev_ptr(logits_out), _dev_ptr(topk_ids),
                                         _dev_ptr(pair_pos), _stream(stream)), "moe_decode_layer_static")


def moe_static_scratch_bytes() -> int:
    return int(lib().moe_static_scratch_bytes())


def moe_combine(ctx: Ctx, y_pairs, topk_w, T: int, k: int, H: int, out, stream=None) -> None:
    _check(lib().moe_combine(ctx.handle, _dev_ptr(y_pairs), _dev_ptr(topk_w), T, k, H, _dev_ptr(out),
                             _stream(stream)), "moe_combine")


def moe_dequantize(ctx: Ctx, qtype: int, packed, rows: int, cols: int, out, stream=None) -> None:
    out_dtype = DTYPE_BF16 if out.dtype == torch.bfloat16 else DTYPE_F32
    _check(lib().moe_dequantize(ctx.handle, qtype, _dev_ptr(packed), rows, cols, out_dtype,
                                _dev_ptr(out), _stream(stream)), "moe_dequantize")


# -------------------------------------------------------------------- cache
class Cache:
    def __init__(self, L, E, n_slots, qtype, H, I, d_pool, h_pool):
        h = ctypes.c_void_p()
        _check(lib().cache_slot_table_create(L, E, n_slots, qtype, H, I, _dev_ptr(d_pool), _ptr(h_pool),
                                             ctypes.byref(h)), "cache_slot_table_create")
        self.handle = h
        self.L, self.E = L, E

    def close(self):
        if self.handle:
            lib().cache_slot_table_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def cache_slot_table_create(L, E, n_slots, qtype, H, I, d_pool, h_pool) -> Cache:
    return Cache(L, E, n_slots, qtype, H, I, d_pool, h_pool)


def cache_slot_table_lookup(cache: Cache, layer: int, ids: Sequence[int]):
    import numpy as np
    a = np.ascontiguousarray(ids, dtype=np.int32)
    n = a.size
    slots = np.empty(n, dtype=np.int32)
    miss = np.empty(max(n, 1), dtype=np.int32)
    nm = ctypes.c_int()
    P = ctypes.POINTER(ctypes.c_int32)
    _check(lib().cache_slot_table_lookup(cache.handle, layer, a.ctypes.data_as(P), n,
                                         slots.ctypes.data_as(P), miss.ctypes.data_as(P),
                                         ctypes.byref(nm)), "cache_slot_table_lookup")
    return slots, miss[: nm.value].copy()


def cache_slot_table_device(cache: Cache) -> int:
    return lib().cache_slot_table_device(cache.handle)


def cache_slot_table_stats(cache: Cache) -> Tuple[int, int]:
    h, m = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().cache_slot_table_stats(cache.handle, ctypes.byref(h), ctypes.byref(m)),
           "cache_slot_table_stats")
    return h.value, m.value


def cache_slot_table_destroy(cache: Cache) -> None:
    cache.close()


def prefetch_expert(cache: Cache, layer: int, expert: int, copy_stream, compute_stream) -> int:
    s = ctypes.c_int32()
    _check(lib().prefetch_expert(cache.handle, layer, expert, _stream(copy_stream),
                                 _stream(compute_stream), ctypes.byref(s)), "prefetch_expert")
    return s.value


def cache_slot_table_resize(cache: Cache, n_slots: int, d_pool=None, stream=None) -> None:
    """New capacity n_slots; d_pool None resizes in place."""
    _check(lib().cache_slot_table_resize(cache.handle, n_slots, None if d_pool is None else _dev_ptr(d_pool),
                                         _stream(stream)), "cache_slot_table_resize")


MISS_COPY, MISS_HOST, MISS_QSTAR, MISS_HOST_COPY = 0, 1, 2, 3


def cache_set_miss_policy(cache: Cache, policy: int, host_threads: int = 0) -> None:
    _check(lib().cache_set_miss_policy(cache.handle, policy, host_threads), "cache_set_miss_policy")


def cache_miss_stats(cache: Cache):
    """(experts copied, experts computed on the host, copy GB/s, host GB/s)."""
    a, b = ctypes.c_int64(), ctypes.c_int64()
    p, h = ctypes.c_double(), ctypes.c_double()
    _check(lib().cache_miss_stats(cache.handle, ctypes.byref(a), ctypes.byref(b), ctypes.byref(p), ctypes.byref(h)),
           "cache_miss_stats")
    return a.value, b.value, p.value, h.value


def cache_last_misses(cache: Cache):
    """(copied expert ids, host expert ids, how many of the host ids were
    misses left out of the cache) of the last cache_decode_layer."""
    import numpy as np
    cp = np.empty(max(cache.E, 1), dtype=np.int32)
    hs = np.empty(max(cache.E, 1), dtype=np.int32)
    nc, nh, no = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    P = ctypes.POINTER(ctypes.c_int32)
    _check(lib().cache_last_misses(cache.handle, cp.ctypes.data_as(P), ctypes.byref(nc), hs.ctypes.data_as(P),
                                   ctypes.byref(nh), ctypes.byref(no)), "cache_last_misses")
    return cp[:nc.value].copy(), hs[:nh.value].copy(), no.value


def cache_mark_layer_done(cache: Cache, layer: int, compute_stream=None) -> None:
    _check(lib().cache_mark_layer_done(cache.handle, layer, _stream(compute_stream)),
           "cache_mark_layer_done")


def cache_decode_layer(cache: Cache, ctx: Ctx, layer: int, x, router_w, bias, logits_in, T: int, k: int,
                       logits_out, topk_ids, topk_w, expert_offsets, sorted_pairs, pair_pos, active, y_pairs,
                       ws, ws_bytes: int, out, copy_stream=None, compute_stream=None) -> None:
    _check(lib().cache_decode_layer(cache.handle, ctx.handle, layer, _dev_ptr(x), _dev_ptr(router_w),
                                    _dev_ptr(bias), _dev_ptr(logits_in), T, k, _dev_ptr(logits_out),
                                    _dev_ptr(topk_ids), _dev_ptr(topk_w), _dev_ptr(expert_offsets),
                                    _dev_ptr(sorted_pairs), _dev_ptr(pair_pos), _dev_ptr(active),
                                    _dev_ptr(y_pairs), _dev_ptr(ws), ws_bytes, _dev_ptr(out),
                                    _stream(copy_stream), _stream(compute_stream)), "cache_decode_layer")


# --------------------------------------------------------- prefill streaming
class PrefillStream:
    def __init__(self, L, E, qtype, H, I, d_bufs, h_pool):
        h = ctypes.c_void_p()
        _check(lib().prefill_stream_create(L, E, qtype, H, I, _dev_ptr(d_bufs), _ptr(h_pool), ctypes.byref(h)),
               "prefill_stream_create")
        self.handle = h

    def close(self):
        if self.handle:
            lib().prefill_stream_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def prefill_stream_create(L, E, qtype, H, I, d_bufs, h_pool) -> PrefillStream:
    return PrefillStream(L, E, qtype, H, I, d_bufs, h_pool)


def prefill_stream_layer(ps: PrefillStream, ctx: Ctx, layer: int, args: moe_ffn_args, router_w, bias, logits_in,
                         logits_out, topk_ids, pair_pos, route_ws, route_ws_bytes: int, copy_stream=None,
                         compute_stream=None) -> None:
    _check(lib().prefill_stream_layer(ps.handle, ctx.handle, layer, ctypes.byref(args), _dev_ptr(router_w),
                                      _dev_ptr(bias), _dev_ptr(logits_in), _dev_ptr(logits_out),
                                      _dev_ptr(topk_ids), _dev_ptr(pair_pos), _dev_ptr(route_ws), route_ws_bytes,
                                      _stream(copy_stream), _stream(compute_stream)), "prefill_stream_layer")


def prefill_stream_stats(ps: PrefillStream) -> Tuple[int, int]:
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().prefill_stream_stats(ps.handle, ctypes.byref(a), ctypes.byref(b)), "prefill_stream_stats")
    return a.value, b.value


def prefill_stream_destroy(ps: PrefillStream) -> None:
    ps.close()


# ------------------------------------------------------------ host executor
def _host_ptr(a) -> int:
    if isinstance(a, torch.Tensor):
        if a.is_cuda:
            raise ValueError("expected a host buffer")
        return _ptr(a)
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("libmoe takes contiguous arrays")
    return a.ctypes.data


def moe_host_expert_ffn(qtype: int, H: int, I: int, slot, x, y, threads: int = 0, vector: bool = True) -> None:
    """Host buffers (numpy or CPU tensors): slot bytes, x fp32 [n, H] -> y fp32 [n, H]."""
    n = int(x.shape[0])
    _check(lib().moe_host_expert_ffn(qtype, H, I, _host_ptr(slot), _host_ptr(x), n, _host_ptr(y), threads,
                                     1 if vector else 0), "moe_host_expert_ffn")


def moe_host_has_avx512() -> bool:
    return bool(lib().moe_host_has_avx512())
