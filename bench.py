#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer forward on one MI355X.

Default workload: decode through 48 stacked, independently weighted MoE
layers (hidden 2048, 128 experts, top-8, intermediate 768, Q8_0 experts,
fp32 activations, every expert resident in HBM), one step = one token batch
through all 48 layers (route -> permute -> expert FFN -> combine per layer),
captured once as a HIP graph and replayed.  `value` is tokens per second
through the stack.

Also reported on the same line:
  roofline      the dominant kernel's algorithmic bytes per launch over its
                average duration, timed with HIP events on its stream
  cpu_baseline  the CPU oracle on a bounded sample of the same workload, on
                every host core (cpu_baselines: every workload, plus
                one-thread figures)
  batches       the same stack at the other batch sizes
  prefill       4096-token grouped-GEMM layer (hidden 2048, 128 experts,
                top-8, intermediate 768, Q4_0, bf16 activations)
  prefill_stream the same layer over 8 layers whose experts stream from
                pinned host memory through two device buffers
  wide          wide-expert decode (hidden 2048, 512 experts, top-10,
                intermediate 512, Q4_0, Zipf-biased router) at 1 and 64
                tokens over 8 layer copies; HBM and fp32-VALU rooflines
  block_types   every block type (Q8_0, Q5_1, Q5_0, Q4_1, Q4_0, Q4_K, Q5_K) on the
                decode shape (8 layers, T=1) and on the prefill layer
  cache         expert-cache decode: 8 layers (hidden 4096, 256 experts,
                top-8, intermediate 2048, Q4_0) served from a pinned host
                pool through a VRAM cache of 40% of the experts, 2048
                single-token steps of a trace with temporal locality; then
                the same trace with misses computed on the host cores
                (all, and split by measured rates: q*), at cache
                fractions 0.1 .. 0.58 (copy and q*), and a run resized
                from 58% to 40% at run time halfway
Progress goes to stderr; the JSON line is the only stdout output.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "MoE-layer tokens/s; decode HBM GB/s and prefill MFMA TFLOP/s as % of peak"


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--batch", type=int, default=1, help="tokens per step of the decode stack")
    p.add_argument("--layers", type=int, default=48)
    p.add_argument("--no-extras", action="store_true", help="skip the other batch sizes, prefill and the expert cache")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-cache", action="store_true", help="skip the expert-cache decode run")
    p.add_argument("--legs", default="batches,wide,prefill,prefill_stream,block_types,cache",
                   help="comma-separated extra legs to run after the headline decode stack")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="first run a device copy and an elementwise negate of MIB MiB each, the known-size "
                        "kernels that scale rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes")
    p.add_argument("--cache-steps", type=int, default=None, help="steps of the expert-cache trace (default 2048)")
    p.add_argument("--sweep-steps", type=int, default=1024,
                   help="steps of each cache-fraction sweep point and of the run-time resize run")
    p.add_argument("--calls", choices=("layer", "two", "four"), default="layer",
                   help="per layer: moe_decode_layer (one call), moe_route_permute + moe_expert_ffn with the "
                        "combine (two), or moe_route, moe_permute, moe_expert_ffn, moe_combine (four)")
    return p.parse_args()


# ---------------------------------------------------------------- decode
class DecodeStack:
    def __init__(self, ctx, wl, n_layers: int, fused="layer", distinct=None):
        import numpy as np
        import torch
        from expert_offload_amd import layer
        from gen import inputs as gi

        self.ctx, self.wl, self.L, self.fused = ctx, wl, n_layers, fused
        self.pool = layer.SlotPool(wl.qtype, wl.H, wl.I, n_layers * wl.E, device="cuda")
        self.perm = [gi.slot_permutation(wl, l) for l in range(n_layers)]
        t0 = time.time()

        if distinct:  # `distinct` generated experts repeated over every slot (timing only)
            made = {}
            gi.generate_blocks_parallel(wl, [(0, e) for e in range(distinct)], lambda l, e, b: made.__setitem__(
                e, layer.pack_expert(wl.qtype, wl.H, wl.I, *b)))
            for slot in range(n_layers * wl.E):
                self.pool.put(slot, made[slot % distinct])
        else:
            def put(l, e, b):
                self.pool.put(l * wl.E + int(self.perm[l][e]), layer.pack_expert(wl.qtype, wl.H, wl.I, *b))

            gi.generate_blocks_parallel(wl, [(l, e) for l in range(n_layers) for e in range(wl.E)], put)
        torch.cuda.synchronize()
        log(f"generated and packed {n_layers}x{wl.E} experts "
            f"({self.pool.data.numel() / 1e9:.1f} GB) in {time.time() - t0:.1f}s")
        self.tables = [torch.from_numpy(p).cuda() for p in self.perm]
        self.router = [torch.from_numpy(gi.router_weight(wl, l)).cuda() for l in range(n_layers)]
        bias = gi.router_bias(wl)
        self.bias = None if bias is None else torch.from_numpy(bias).cuda()
        self.np = np

    mode = 0  # MOE_MODE_DECODE; MOE_MODE_DECODE_Q8A for int8 activations

    def buffers(self, T):
        from expert_offload_amd import layer
        wl = self.wl
        return [layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device="cuda", mode=self.mode)
                for _ in range(self.L)]

    def run(self, bufs, x, stream=None):
        from expert_offload_amd import layer
        wl = self.wl
        for l in range(self.L):
            layer.forward(self.ctx, bufs[l], self.pool.base(l * wl.E), self.pool.slot_bytes, wl.E,
                          self.tables[l], x, router_w=self.router[l], bias=self.bias, stream=stream,
                          fused=self.fused)

    def n_active(self, bufs):
        return [int(b.active[0].item()) for b in bufs]


def time_graph(stack, T, steps, warmup):
    import torch
    from gen import inputs as gi
    x = torch.from_numpy(gi.activations(stack.wl, T)).cuda()
    bufs = stack.buffers(T)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        stack.run(bufs, x)  # eager warm-up outside the capture
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        stack.run(bufs, x)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    stack.last_replay_ms = {"median": float(sorted(per)[steps // 2]), "mean": sum(per) / steps,
                            "min": min(per), "max": max(per)}
    return x, bufs, wall, ev[0].elapsed_time(ev[-1])


def kernel_profile(stack, x, bufs, reps=5, names=("router_logits", "topk_permute", "topk", "permute", "ffn_gateup",
                                                  "ffn_gateup_mfma", "ffn_down", "ffn_down_mfma", "combine")):
    """Per-kernel average durations from the library's event timing (eager)."""
    import torch
    import expert_offload_amd as moe
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        stack.run(bufs, x)
    s.synchronize()
    moe.moe_ctx_set_timing(stack.ctx, True)
    with torch.cuda.stream(s):
        for _ in range(reps):
            stack.run(bufs, x)
    s.synchronize()
    out = {}
    for name in names:
        n, ms = moe.moe_ctx_kernel_time(stack.ctx, name)
        if n:
            out[name] = (n, ms)
    moe.moe_ctx_set_timing(stack.ctx, False)
    return out


def decode_kernel_bytes(wl, T, n_active_per_layer):
    """Algorithmic bytes per launch (averaged over layers) of the FFN kernels."""
    from gen import inputs as gi
    qb = gi.BLOCK_BYTES[wl.qtype] / 32.0
    gate_up = 2 * wl.I * wl.H * qb
    down = wl.H * wl.I * qb
    na = sum(n_active_per_layer) / len(n_active_per_layer)
    return {
        "ffn_gateup": na * gate_up + T * wl.H * 4,
        "ffn_down": na * down + T * wl.H * 4,
    }


def decode_layer_bytes(wl, T, n_active):
    from gen import inputs as gi
    return n_active * gi.bytes_per_expert(wl) + wl.E * wl.H * 4 + 2 * T * wl.H * 4


# ---------------------------------------------------------------- prefill
def types_extra(ctx, layers=8, steps=40, warmup=5):
    """Every block type on the decode shape (hidden 2048, 128 experts, top-8,
    intermediate 768, T=1; 8 layers from 32 generated experts repeated,
    since values do not change the timing) and on the 4096-token prefill
    layer: time per decode layer and its algorithmic bytes over that time,
    and the prefill FFN TFLOP/s."""
    import dataclasses
    import torch
    from gen import inputs as gi
    out = {}
    for qt in ("q8_0", "q5_1", "q5_0", "q4_1", "q4_0", "q4_k", "q5_k"):
        wl = dataclasses.replace(gi.workload("decode_q8_0_h2048_e128"), qtype=qt, name=f"decode_{qt}_h2048_e128")
        stack = DecodeStack(ctx, wl, layers, distinct=32)
        x, bufs, _, gpu_ms = time_graph(stack, 1, steps, warmup)
        ms = gpu_ms / steps
        na = stack.n_active(bufs)
        layer_bytes = sum(decode_layer_bytes(wl, 1, a) for a in na) / len(na)
        res = {"decode_layer_us": ms / layers * 1e3, "decode_tokens_per_s_per_layer": layers / (ms * 1e-3),
               "decode_layer_hbm_gbs": layer_bytes / (ms / layers * 1e-3) / 1e9,
               "bytes_per_expert": gi.bytes_per_expert(wl)}
        del stack, bufs, x
        torch.cuda.empty_cache()
        pf = prefill_extra(ctx, steps=5, warmup=2, qtype=qt)
        res["prefill_tokens_per_s"] = pf["tokens_per_s"]
        res["prefill_ffn_tflops"] = pf["ffn_tflops"]
        out[qt] = res
        log(f"type {qt}: decode {ms / layers * 1e3:.1f} us/layer ({res['decode_layer_hbm_gbs']:.0f} GB/s over the "
            f"layer); prefill {pf['tokens_per_s']:.0f} tok/s, FFN {pf['ffn_tflops']:.0f} TFLOP/s")
        torch.cuda.empty_cache()
    return out


def prefill_extra(ctx, steps=10, warmup=3, qtype=None):
    import numpy as np
    import torch
    import expert_offload_amd as moe
    from expert_offload_amd import _lib as L
    from expert_offload_amd import layer
    from gen import inputs as gi

    wl = gi.workload("prefill_q4_0_h2048_e128")
    if qtype:
        import dataclasses
        wl = dataclasses.replace(wl, qtype=qtype, name=f"prefill_{qtype}_h2048_e128")
    T = wl.batches[0]
    pool = layer.SlotPool(wl.qtype, wl.H, wl.I, wl.E, device="cuda")
    perm = gi.slot_permutation(wl, 0)

    def put(l, e, b):
        pool.put(int(perm[e]), layer.pack_expert(wl.qtype, wl.H, wl.I, *b))

    gi.generate_blocks_parallel(wl, [(0, e) for e in range(wl.E)], put)
    table = torch.from_numpy(perm).cuda()
    xbits = gi.activations(wl, T)
    x = torch.from_numpy(xbits.view(np.int16)).view(torch.bfloat16).cuda()
    logits = torch.from_numpy(gi.given_logits(wl, T)).cuda()
    buf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device="cuda",
                             mode=L.MODE_PREFILL, x_dtype=L.DTYPE_BF16)

    def run():
        layer.forward(ctx, buf, pool.base(), pool.slot_bytes, wl.E, table, x, logits_in=logits)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        run()
    ev1.record()
    torch.cuda.synchronize()
    ms_eager = ev0.elapsed_time(ev1) / steps
    # The same layer as a HIP graph, as a serving loop would issue it (no
    # launch gaps between its kernels).  Every replay's output is checked bit
    # for bit against the eager one, with eager forwards between replays.
    out_eager = buf.out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    graph_ok = True
    for _ in range(3):
        buf.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        graph_ok &= bool(torch.equal(buf.out, out_eager))
        run()
        torch.cuda.synchronize()
        graph_ok &= bool(torch.equal(buf.out, out_eager))
    if not graph_ok:
        raise RuntimeError("prefill layer: a graph replay differs from the eager forward")
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    ms = ev[0].elapsed_time(ev[-1]) / steps
    graph_ok &= bool(torch.equal(buf.out, out_eager))
    if not graph_ok:
        raise RuntimeError("prefill layer: a graph replay differs from the eager forward")
    moe.moe_ctx_set_timing(ctx, True)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    kt = {}
    for name in ("topk", "permute", "permute_count", "permute_scan", "permute_scatter", "ffn_gateup", "ffn_down",
                 "combine"):
        n, t = moe.moe_ctx_kernel_time(ctx, name)
        if n:
            kt[name] = t / n
    moe.moe_ctx_set_timing(ctx, False)
    flops = 2.0 * T * wl.k * 3 * wl.H * wl.I
    gu_ms = kt.get("ffn_gateup", 0)
    ffn_ms = gu_ms + kt.get("ffn_down", 0)
    tflops = flops / (ffn_ms * 1e-3) / 1e12 if ffn_ms else None
    gate_up_flops = 2.0 * T * wl.k * 2 * wl.H * wl.I
    gu_tflops = gate_up_flops / (gu_ms * 1e-3) / 1e12 if gu_ms else None
    return {
        "workload": wl.name, "tokens": T, "layer_ms": ms, "tokens_per_s": T / (ms * 1e-3),
        "timing": "hip graph of the layer, replayed; every replay equal bit for bit to the eager forward",
        "median_layer_ms": per[steps // 2], "layer_ms_eager": ms_eager, "tokens_per_s_eager": T / (ms_eager * 1e-3),
        "kernel_ms": kt, "ffn_tflops": tflops, "ffn_frac_bf16_peak": tflops / BF16_PEAK_TFLOPS if tflops else None,
        "gateup_tflops": gu_tflops,
        "flops_per_layer": flops,
    }


# ---------------------------------------------------------------- wide experts
VALU_F32_PEAK_TFLOPS = 157.3


def wide_extra(ctx, layers=8, steps=30, warmup=5, distinct=128):
    """Wide-expert decode: hidden 2048, 512 experts, top-10, intermediate
    512, Q4_0 experts, fp32 router 2048x512 with the Zipf(1.1) logit bias,
    at 1 and 64 tokens.  `layers` independently routed layer copies (906 MB
    of experts each, 7.2 GB for 8) are run in turn, one moe_decode_layer call
    each, as one HIP graph, so no layer's experts are still in the 256 MB
    MALL when it comes round again.  The pool holds `distinct` generated
    experts repeated over the slots (the bytes read per layer and the
    routing are the workload's; the values do not change the timing)."""
    import dataclasses
    import torch
    from gen import inputs as gi

    wl = dataclasses.replace(gi.workload("wide_q4_0_h2048_e512"), layers=layers)
    stack = DecodeStack(ctx, wl, layers, distinct=distinct)
    out = {"workload": f"{wl.name} x {layers} layer copies", "layers": layers,
           "expert_bytes_per_layer": wl.E * gi.bytes_per_expert(wl),
           "pool_values": f"{distinct} generated experts repeated over the {layers * wl.E} slots"}
    for T in wl.batches:
        x, bufs, wall, _ = time_graph(stack, T, steps, warmup)
        ms = wall * 1e3 / steps
        layer_us = ms / layers * 1e3
        na = stack.n_active(bufs)
        prof = kernel_profile(stack, x, bufs)
        kb = decode_kernel_bytes(wl, T, na)
        layer_bytes = sum(decode_layer_bytes(wl, T, a) for a in na) / len(na)
        flops = 2.0 * T * wl.k * 3 * wl.H * wl.I
        kus = {name: ms_ / n * 1e3 for name, (n, ms_) in prof.items()}
        ffn_us = sum(kus.get(n_, 0) for n_ in ("ffn_gateup", "ffn_gateup_mfma", "ffn_down", "ffn_down_mfma"))
        res = {"tokens": T, "tokens_per_s_per_layer": T / (layer_us * 1e-6), "layer_us": layer_us,
               "median_layer_us": stack.last_replay_ms["median"] / layers * 1e3,
               "mean_active_experts": sum(na) / len(na), "layer_bytes": layer_bytes,
               "layer_hbm_gbs": layer_bytes / (layer_us * 1e-6) / 1e9,
               "layer_hbm_frac": layer_bytes / (layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
               "kernel_us": kus,
               "ffn_flops": flops,
               # the fp32 FFN arithmetic over the GEMV and matrix-core kernels together
               "ffn_fp32_tflops": flops / (ffn_us * 1e-6) / 1e12,
               "ffn_fp32_frac": flops / (ffn_us * 1e-6) / 1e12 / VALU_F32_PEAK_TFLOPS,
               "ffn_hbm_frac": (kb["ffn_gateup"] + kb["ffn_down"]) / (ffn_us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        for part in ("gateup", "down"):  # both kernels of a part (matrix-core experts, the others)
            t_ = kus.get("ffn_" + part, 0) + kus.get("ffn_%s_mfma" % part, 0)
            res[part + "_hbm_frac"] = kb["ffn_" + part] / (t_ * 1e-6) / 1e9 / HBM_PEAK_GBS
        # which roofline binds: the larger of the two times at peak (the fp32
        # peak is the same for the VALU and the fp32 matrix cores)
        t_hbm = (kb["ffn_gateup"] + kb["ffn_down"]) / (HBM_PEAK_GBS * 1e9)
        t_valu = flops / (VALU_F32_PEAK_TFLOPS * 1e12)
        res["ffn_bound"] = "hbm" if t_hbm >= t_valu else "fp32 arithmetic"
        res["ffn_floor_us"] = {"hbm": t_hbm * 1e6, "valu_fp32": t_valu * 1e6}
        # the same layers with int8 activations (MOE_MODE_DECODE_Q8A)
        from expert_offload_amd import _lib as L
        stack.mode = L.MODE_DECODE_Q8A
        xq, bq, wq, _ = time_graph(stack, T, steps, warmup)
        kq = kernel_profile(stack, xq, bq, names=("router_logits", "topk_permute", "topk", "permute", "quant_act",
                                                   "ffn_gateup", "ffn_down"))
        stack.mode = 0
        q_us = wq * 1e3 / steps / layers * 1e3
        res["int8_activations"] = {"layer_us": q_us, "tokens_per_s_per_layer": T / (q_us * 1e-6),
                                   "kernel_us": {n: ms_ / c * 1e3 for n, (c, ms_) in kq.items()}}
        out[str(T)] = res
        log(f"wide T={T}: {layer_us:.1f} us/layer ({res['tokens_per_s_per_layer']:.0f} tok/s per layer), "
            f"{res['mean_active_experts']:.1f} experts, layer {res['layer_hbm_gbs']:.0f} GB/s; kernels "
            + ", ".join(f"{k_} {v:.1f}" for k_, v in kus.items()) + f" us; FFN bound {res['ffn_bound']}; "
            f"int8 activations {q_us:.1f} us/layer ("
            + ", ".join(f"{k_} {v:.1f}" for k_, v in res["int8_activations"]["kernel_us"].items()) + " us)")
        del bufs, x, bq, xq
    del stack
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- prefill streaming
def prefill_stream_extra(ctx, layers=8, reps=3):
    """The 4096-token prefill layer (hidden 2048, 128 experts, top-8,
    intermediate 768, Q4_0) over `layers` layers whose experts all live in
    pinned host memory: each layer's 339.7 MB of experts crosses PCIe into
    one of two device buffers while the previous layer computes.  Timed
    beside it: the copies alone, the layers alone (experts resident), and
    copy-then-compute with no overlap.

    Every layer's host experts are the bytes of one generated layer; the
    copy and FFN times do not depend on the values, while the routing
    (given logits) differs per layer.  Parity of this path is covered by
    the tests."""
    import dataclasses
    import numpy as np
    import torch
    import expert_offload_amd as moe
    from expert_offload_amd import _lib as L
    from expert_offload_amd import layer
    from gen import inputs as gi

    wl = dataclasses.replace(gi.workload("prefill_q4_0_h2048_e128"), layers=layers)
    T = wl.batches[0]
    q = L.QTYPE[wl.qtype]
    sb = moe.moe_slot_bytes(q, wl.H, wl.I)
    lb = wl.E * sb
    pool = torch.empty(layers * lb, dtype=torch.uint8, pin_memory=True)
    view = pool.numpy()
    one = np.empty(lb, dtype=np.uint8)

    def put(l, e, b):
        one[e * sb:(e + 1) * sb] = layer.pack_expert(wl.qtype, wl.H, wl.I, *b)

    gi.generate_blocks_parallel(wl, [(0, e) for e in range(wl.E)], put)
    for l in range(layers):
        view[l * lb:(l + 1) * lb] = one
    xd = torch.from_numpy(gi.activations(wl, T).view(np.int16)).view(torch.bfloat16).cuda()
    logits = [torch.from_numpy(gi.given_logits(wl, T, l)).cuda() for l in range(layers)]
    sp = layer.StreamedPrefill(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, layers, T, pool)
    s = torch.cuda.current_stream()

    def timed(fn, stream=None):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def streamed():
        for l in range(layers):
            sp.layer(l, xd, logits[l])

    def copies():
        with torch.cuda.stream(sp.copy_stream):
            for l in range(layers):
                b = l % 2
                sp.d_bufs[b * lb:(b + 1) * lb].copy_(pool[l * lb:(l + 1) * lb], non_blocking=True)

    ident = torch.arange(wl.E, dtype=torch.int32, device="cuda")
    rbuf = layer.LayerBuffers(T, wl.H, wl.I, wl.E, wl.k, wl.qtype, device="cuda", mode=L.MODE_PREFILL,
                              x_dtype=L.DTYPE_BF16)

    def computes(copy_first=False):
        for l in range(layers):
            if copy_first:  # on the compute stream: no overlap
                sp.d_bufs[:lb].copy_(pool[l * lb:(l + 1) * lb], non_blocking=True)
            layer.forward(ctx, rbuf, sp.d_bufs.data_ptr(), sb, wl.E, ident, xd, logits_in=logits[l], fused=True)

    streamed()
    computes()
    t_stream = min(timed(streamed) for _ in range(reps))
    t_copy = min(timed(copies, sp.copy_stream) for _ in range(reps))
    t_compute = min(timed(computes) for _ in range(reps))
    t_serial = min(timed(lambda: computes(True)) for _ in range(reps))
    moe.moe_ctx_check(ctx)
    loads, demand = sp.stats()
    sp.close()
    del sp, pool, rbuf
    torch.cuda.empty_cache()
    hidden = t_copy + t_compute - t_stream
    return {
        "workload": f"{wl.name} x {layers} layers streamed", "tokens": T, "layers": layers,
        "layer_expert_bytes": lb, "host_pool_bytes": layers * lb,
        "tokens_per_s": T * layers / (t_stream * 1e-3), "ms_per_layer": t_stream / layers,
        "h2d_gbs": layers * lb / (t_stream * 1e-3) / 1e9,
        "copy_only_ms_per_layer": t_copy / layers, "copy_only_gbs": layers * lb / (t_copy * 1e-3) / 1e9,
        "compute_only_ms_per_layer": t_compute / layers, "serial_ms_per_layer": t_serial / layers,
        "speedup_vs_serial": t_serial / t_stream,
        "overlap_efficiency": hidden / min(t_copy, t_compute),
        "copies": loads, "demand_loads": demand,
        "pool_values": "one generated layer's experts repeated over the layers",
    }


# ---------------------------------------------------------------- expert cache
SWEEP_FRACTIONS = (0.1, 0.2, 0.3, 0.4, 0.5, 0.58)


def cache_extra(ctx, steps=None, distinct=64, warm_from=256, sweep_steps=1024, resize_from=0.58):
    """Expert-cache decode: 8 layers (hidden 4096, 256 experts, top-8,
    intermediate 2048, Q4_0), the whole pool in pinned host memory, a VRAM
    cache of 40% of each layer's experts (816 slots), single-token steps
    following a trace with temporal locality, from an empty cache.

    Then, on the same trace: `sweep_steps` steps at each cache fraction of
    SWEEP_FRACTIONS, and one run that starts at `resize_from` and resizes the
    cache to the main run's fraction at run time halfway (a new, smaller
    pool; the kept experts move on device).

    The pinned pool holds `distinct` generated experts repeated over the
    2048 (layer, expert) keys: the bytes moved and read are those of the
    workload, and the copy and FFN times do not depend on the values
    (parity of this path is covered by the tests)."""
    import numpy as np
    import torch
    import expert_offload_amd as moe
    from expert_offload_amd import _lib as L
    from expert_offload_amd import layer
    from gen import inputs as gi

    wl = gi.workload("cache_q4_0_h4096_e256")
    steps = steps or wl.steps
    q = L.QTYPE[wl.qtype]
    sb = moe.moe_slot_bytes(q, wl.H, wl.I)
    keys = wl.layers * wl.E
    n_slots = int(wl.cache_fraction * wl.E) * wl.layers
    log(f"cache: pinning a {keys * sb / 1e9:.1f} GB host pool ({keys} experts of {sb} B)")
    pool = torch.empty(keys * sb, dtype=torch.uint8, pin_memory=True)
    base = {}
    gi.generate_blocks_parallel(wl, [(b // wl.E, b % wl.E) for b in range(distinct)],
                                lambda l, e, b: base.__setitem__(l * wl.E + e, layer.pack_expert(
                                    wl.qtype, wl.H, wl.I, *b)))
    view = pool.numpy()
    for key in range(keys):
        view[key * sb:(key + 1) * sb] = base[key % distinct]
    del base
    log("cache: pool filled; building the trace")
    n_trace = max(steps, sweep_steps)
    trace = gi.cache_trace(wl, n_trace)
    logits = torch.from_numpy(np.stack([gi.cache_trace_logits(wl, trace, s) for s in range(n_trace)])).cuda()
    xs = torch.from_numpy(np.stack([gi.activations(wl, 1, s)[0] for s in range(n_trace)])).cuda()

    def run(cl, s0, s1, tag):
        """Steps [s0, s1); wall-clock stamp after each step's host calls."""
        torch.cuda.synchronize()
        stamps = [time.perf_counter()]
        for s in range(s0, s1):
            x = xs[s:s + 1]
            for l in range(wl.layers):
                cl.layer(l, x, logits[s, l:l + 1])
            stamps.append(time.perf_counter())
            if (s + 1 - s0) % 512 == 0:
                log(f"cache {tag}: step {s + 1 - s0}/{s1 - s0}")
        torch.cuda.synchronize()
        stamps[-1] = time.perf_counter()
        moe.moe_ctx_check(ctx)
        return stamps

    def phase(cl, stamps, s0, s1, w0):
        """tokens/s and hit rate over steps [w0, s1) of a run that began at s0."""
        mpl = np.array(cl.misses_per_layer[(w0 - s0) * wl.layers:(s1 - s0) * wl.layers])
        return {"steps": [w0, s1], "tokens_per_s": (s1 - w0) / (stamps[s1 - s0] - stamps[w0 - s0]),
                "hit_rate": 1.0 - float(mpl.sum()) / ((s1 - w0) * wl.layers * wl.k)}

    def slots_of(f):
        return int(f * wl.E) * wl.layers

    cl = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, n_slots, pool)
    stamps = run(cl, 0, steps, "main")
    wall = stamps[-1] - stamps[0]
    hits, misses = cl.stats()
    main_misses = list(cl.misses_per_layer)
    warm = phase(cl, stamps, 0, steps, min(warm_from, steps - 1))
    # PCIe ceiling: back-to-back expert copies from the pinned pool
    cs = torch.cuda.Stream()
    d = cl.d_pool
    n_cp = 32
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cs):
        e0.record()
        for i in range(n_cp):
            j = (i * 37) % keys
            d[(i % n_slots) * sb:(i % n_slots + 1) * sb].copy_(pool[j * sb:(j + 1) * sb], non_blocking=True)
        e1.record()
    torch.cuda.synchronize()
    ceiling = n_cp * sb / (e0.elapsed_time(e1) * 1e-3) / 1e9
    cl.close()
    del cl, d
    torch.cuda.empty_cache()
    res = {
        "workload": wl.name, "layers": wl.layers, "steps": steps, "cache_slots": n_slots,
        "cache_fraction": wl.cache_fraction, "expert_bytes": sb, "host_pool_bytes": keys * sb,
        "tokens_per_s": steps / wall, "ms_per_token": wall * 1e3 / steps,
        "hit_rate": hits / (hits + misses),
        "warm": {"from_step": warm["steps"][0], "tokens_per_s": warm["tokens_per_s"], "hit_rate": warm["hit_rate"]},
        "h2d_gbs": misses * sb / wall / 1e9,
        "h2d_copy_ceiling_gbs": ceiling,
        "pool_values": f"{distinct} generated experts repeated over the {keys} keys",
        "_misses_per_layer": main_misses,
    }
    # misses on the host cores (MOE_MISS_HOST) and split by measured rates
    # (MOE_MISS_QSTAR), same trace and cache size
    for name, pol in (("host", L.MISS_HOST), ("qstar", L.MISS_QSTAR), ("host_copy", L.MISS_HOST_COPY)):
        cl = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, n_slots, pool)
        cl.set_miss_policy(pol)
        st = run(cl, 0, steps, name)
        ph = phase(cl, st, 0, steps, min(warm_from, steps - 1))
        copied, on_host, r_copy, r_host = cl.miss_stats()
        res[name] = {"tokens_per_s": steps / (st[-1] - st[0]), "warm": ph,
                     "hit_rate": 1.0 - float(sum(cl.misses_per_layer)) / (steps * wl.layers * wl.k),
                     "experts_copied": copied, "experts_on_host": on_host,
                     "copy_gbs_estimate": r_copy, "host_gbs_estimate": r_host,
                     "host_threads": "all hardware threads but four"}
        log(f"cache {name}: {res[name]['tokens_per_s']:.1f} tok/s (warm {ph['tokens_per_s']:.1f} at hit rate "
            f"{ph['hit_rate']:.3f}); copied {copied}, on host {on_host}; rates copy {r_copy:.1f} host "
            f"{r_host:.1f} GB/s")
        cl.close()
        del cl
        torch.cuda.empty_cache()
    # cache-fraction sweep, each from an empty cache over the first sweep_steps steps
    sweep = []
    w0 = min(warm_from, sweep_steps - 1)
    for f in SWEEP_FRACTIONS:
        cl = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, slots_of(f), pool)
        st = run(cl, 0, sweep_steps, f"{f:.2f}")
        ph = phase(cl, st, 0, sweep_steps, w0)
        late = phase(cl, st, 0, sweep_steps, sweep_steps // 2)
        point = {"cache_fraction": f, "cache_slots": slots_of(f), "tokens_per_s": ph["tokens_per_s"],
                 "hit_rate": ph["hit_rate"], "from_step": w0, "second_half": late}
        cl.close()
        del cl
        torch.cuda.empty_cache()
        msg = ""
        for name, pol in (("qstar", L.MISS_QSTAR), ("host_copy", L.MISS_HOST_COPY)):
            cl = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, slots_of(f), pool)
            cl.set_miss_policy(pol)
            st = run(cl, 0, sweep_steps, f"{f:.2f} {name}")
            qph = phase(cl, st, 0, sweep_steps, w0)
            point[name] = {"tokens_per_s": qph["tokens_per_s"], "hit_rate": qph["hit_rate"],
                           "experts_on_host": cl.miss_stats()[1]}
            msg += f"; {name} {qph['tokens_per_s']:.1f} tok/s at {qph['hit_rate']:.3f}"
            cl.close()
            del cl
            torch.cuda.empty_cache()
        sweep.append(point)
        log(f"cache sweep {f:.2f}: {ph['tokens_per_s']:.1f} tok/s at hit rate {ph['hit_rate']:.3f}{msg}")
    res["sweep"] = {"steps": sweep_steps, "points": sweep}
    # run-time resize from resize_from to the main fraction, halfway through
    half = sweep_steps // 2
    cl = layer.CachedLayers(ctx, wl.qtype, wl.H, wl.I, wl.E, wl.k, wl.layers, slots_of(resize_from), pool)
    st1 = run(cl, 0, half, "before resize")
    before = phase(cl, st1, 0, half, min(w0, half - 1))
    t0 = time.perf_counter()
    cl.resize(slots_of(wl.cache_fraction))
    torch.cuda.synchronize()
    resize_ms = (time.perf_counter() - t0) * 1e3
    cl.misses_per_layer = []
    st2 = run(cl, half, sweep_steps, "after resize")
    after = phase(cl, st2, half, sweep_steps, half)
    cl.close()
    del cl
    torch.cuda.empty_cache()
    res["resize"] = {"from_fraction": resize_from, "to_fraction": wl.cache_fraction,
                     "from_slots": slots_of(resize_from), "to_slots": slots_of(wl.cache_fraction),
                     "at_step": half, "resize_ms": resize_ms, "before": before, "after": after,
                     "after_vs_before": after["tokens_per_s"] / before["tokens_per_s"]}
    fixed = [p["second_half"] for p in sweep if p["cache_fraction"] == wl.cache_fraction]
    if fixed:  # the same steps at a cache that was never resized
        res["resize"]["after_vs_fixed"] = after["tokens_per_s"] / fixed[0]["tokens_per_s"]
    log(f"cache resize {resize_from:.2f} -> {wl.cache_fraction:.2f}: {resize_ms:.1f} ms; "
        f"{before['tokens_per_s']:.1f} -> {after['tokens_per_s']:.1f} tok/s")
    del pool
    return res


# ---------------------------------------------------------------- CPU oracle
def host_threads() -> int:
    """The host cores this process may use (at most 16: the GPU machine's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _oracle_jobs_rate(jobs, threads):
    """Runs `jobs` (callables, each one oracle layer forward returning the
    tokens it processed) on `threads` worker threads, BLAS held to one
    thread per worker; returns (tokens, seconds)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if threads == 1:
            toks = sum(f() for f in jobs)
        else:
            with ThreadPoolExecutor(threads) as ex:
                toks = sum(ex.map(lambda f: f(), jobs))
        return toks, time.perf_counter() - t0


def _oracle_decode_jobs(wl, T, n_jobs, distinct=16):
    """n_jobs oracle layer forwards of a decode workload (layer l = job mod
    layers: its router and x); expert blocks are `distinct` generated ones
    repeated over the ids (the oracle's cost does not depend on the values)."""
    from gen import inputs as gi
    import oracle
    blocks = {}
    gi.generate_blocks_parallel(wl, [(0, e) for e in range(min(distinct, wl.E))],
                                lambda l, e, b: blocks.__setitem__(e, b))
    pool = [blocks[e] for e in sorted(blocks)]
    x = gi.activations(wl, T)
    bias = gi.router_bias(wl)
    routers = {l: gi.router_weight(wl, l) for l in range(min(n_jobs, wl.layers))}

    def job(l):
        def run():
            oracle.moe_layer(x, wl.qtype, lambda e: pool[(l * 7 + e) % len(pool)], wl.k,
                             router_w=routers[l], bias=bias)
            return T
        return run
    return [job(j % len(routers)) for j in range(n_jobs)]


def cpu_baselines(gpu_cache_misses=None):
    """The CPU oracle (NumPy, float64) timed on this host's cores for every
    workload: decode workloads as concurrent layer forwards, one per worker
    thread (whole-job throughput of independent sequences), the prefill
    layer with BLAS on every thread, the expert-cache workload as layer
    forwards plus its full LRU simulation.  Also one-thread figures for the
    tiny layer and the decode stack at one token."""
    import dataclasses
    import numpy as np
    from threadpoolctl import threadpool_limits
    from gen import inputs as gi
    import oracle

    threads = host_threads()
    model = cpu_model()
    out = {"cores": threads, "cpu_model": model, "kind": "oracle"}

    def entry(name, wl, T, n_jobs, per="layer", threads_=threads):
        toks, sec = _oracle_jobs_rate(_oracle_decode_jobs(wl, T, n_jobs), threads_)
        r = {"tokens_per_s_per_layer": toks / sec, "layer_forwards": n_jobs, "seconds": sec,
             "threads": threads_}
        if wl.layers > 1:
            r["tokens_per_s_stack"] = toks / sec / wl.layers
        log(f"cpu oracle {name}: {toks / sec:.2f} tok/s per layer on {threads_} threads ({n_jobs} layer forwards "
            f"in {sec:.1f}s)")
        return r

    tiny = gi.workload("tiny_q8_0")
    dec = gi.workload("decode_q8_0_h2048_e128")
    wide = gi.workload("wide_q4_0_h2048_e512")
    out["tiny_q8_0 T=4"] = entry("tiny T=4", tiny, 4, 4096)
    out["tiny_q8_0 T=4 1 thread"] = entry("tiny T=4 (1 thread)", tiny, 4, 1024, threads_=1)
    out["decode_q8_0_h2048_e128 T=1"] = entry("decode T=1", dec, 1, 480)
    out["decode_q8_0_h2048_e128 T=1 1 thread"] = entry("decode T=1 (1 thread)", dec, 1, 48, threads_=1)
    out["decode_q8_0_h2048_e128 T=4"] = entry("decode T=4", dec, 4, 96)
    out["decode_q8_0_h2048_e128 T=16"] = entry("decode T=16", dec, 16, 48)
    out["wide_q4_0_h2048_e512 T=1"] = entry("wide T=1", wide, 1, 320)
    out["wide_q4_0_h2048_e512 T=64"] = entry("wide T=64", wide, 64, 48)
    # prefill: one 4096-token layer, BLAS on every thread
    pf = gi.workload("prefill_q4_0_h2048_e128")
    T = pf.batches[0]
    blocks = {}
    gi.generate_blocks_parallel(pf, [(0, e) for e in range(16)], lambda l, e, b: blocks.__setitem__(e, b))
    pool = [blocks[e] for e in sorted(blocks)]
    x32 = gi.bf16_bits_to_f32(gi.activations(pf, T))
    logits = gi.given_logits(pf, T)
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        oracle.moe_layer(x32, pf.qtype, lambda e: pool[e % len(pool)], pf.k, logits=logits)
        sec = time.perf_counter() - t0
    out["prefill_q4_0_h2048_e128 T=4096"] = {"tokens_per_s_per_layer": T / sec, "seconds": sec, "threads": threads,
                                             "blas_threads": threads}
    log(f"cpu oracle prefill T={T}: {T / sec:.0f} tok/s per layer ({sec:.1f}s, BLAS on {threads} threads)")
    # expert cache: layer forwards of the trace's routing, and the LRU over the whole trace
    cw = gi.workload("cache_q4_0_h4096_e256")
    trace = gi.cache_trace(cw)
    cblocks = {}
    gi.generate_blocks_parallel(cw, [(0, e) for e in range(8)], lambda l, e, b: cblocks.__setitem__(e, b))
    cpool = [cblocks[e] for e in sorted(cblocks)]
    n_jobs = 64
    lg = [gi.cache_trace_logits(cw, trace, s) for s in range(n_jobs // cw.layers)]

    def cjob(j):
        s_, l = j // cw.layers, j % cw.layers

        def run():
            x = gi.activations(cw, 1, s_)
            oracle.moe_layer(x, cw.qtype, lambda e: cpool[e % len(cpool)], cw.k, logits=lg[s_][l:l + 1])
            return 1
        return run
    toks, sec = _oracle_jobs_rate([cjob(j) for j in range(n_jobs)], threads)
    order = np.stack([oracle.topk_select(gi.cache_trace_logits(cw, trace, s), cw.k) for s in range(trace.shape[0])])
    t0 = time.perf_counter()
    hit, _ = oracle.lru_simulate(order, int(cw.cache_fraction * cw.E) * cw.layers)
    lru_s = time.perf_counter() - t0
    ce = {"tokens_per_s": toks / sec / cw.layers, "layer_forwards": n_jobs, "seconds": sec, "threads": threads,
          "lru_seconds": lru_s, "lru_hit_rate": float(hit.mean()),
          "note": "the host holds every expert, so the oracle needs no cache; its LRU is simulated over the "
                  "whole trace only to check the GPU run's misses"}
    if gpu_cache_misses is not None:
        want = (~hit).sum(axis=2).reshape(-1)
        got = np.asarray(gpu_cache_misses)
        ce["gpu_misses_per_layer_match"] = bool(got.shape == want.shape and np.array_equal(got, want))
    out["cache_q4_0_h4096_e256 T=1"] = ce
    log(f"cpu oracle cache: {ce['tokens_per_s']:.3f} tok/s; LRU over {trace.shape[0]} steps in {lru_s:.1f}s, "
        f"hit rate {hit.mean():.4f}" + (f", GPU misses per layer match: {ce['gpu_misses_per_layer_match']}"
                                        if gpu_cache_misses is not None else ""))
    return out


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the layer runs on one GPU; how it would shard is described, not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch
    import expert_offload_amd as moe
    from gen import inputs as gi

    from expert_offload_amd.rocprof_summary import traffic_bytes
    moe.lib()
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy calibration: {n * 4} B copied and negated 3 times")
        del src, dst
    wl = gi.workload("decode_q8_0_h2048_e128")
    if args.layers != wl.layers:
        log(f"NOTE: {args.layers} layers instead of {wl.layers} (profiling run)")
    ctx = moe.Ctx(0)
    stack = DecodeStack(ctx, wl, args.layers, fused={"layer": "layer", "two": True, "four": False}[args.calls])

    T = args.batch
    x, bufs, wall, gpu_ms = time_graph(stack, T, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    n_active = stack.n_active(bufs)
    moe.moe_ctx_check(ctx)
    log(f"T={T}: {ms_per_step:.3f} ms/step wall, {gpu_ms / args.steps:.3f} ms/step GPU, "
        f"{T / (ms_per_step * 1e-3):.1f} tok/s, mean active experts {sum(n_active) / len(n_active):.1f}")

    prof = kernel_profile(stack, x, bufs)
    kbytes = decode_kernel_bytes(wl, T, n_active)
    ffn = {k: v for k, v in prof.items() if k in kbytes}
    dom = max(ffn, key=lambda k: ffn[k][1])
    n, tot = ffn[dom]
    avg_ms = tot / n
    achieved = kbytes[dom] / (avg_ms * 1e-3) / 1e9
    for name, (cnt, ms) in sorted(prof.items()):
        log(f"   kernel {name:14s} launches {cnt:5d} avg {ms / cnt * 1e3:8.2f} us")
    rp_kernel = {"ffn_gateup": "ffn_gateup_decode", "ffn_down": "ffn_down_decode"}[dom]
    traffic = traffic_bytes(rp_kernel, os.path.join(ROOT, "profiles", f"{rp_kernel}_h2048_e128_t{T}_traffic.txt"))
    roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "avg_us": avg_ms * 1e3,
                "bytes_per_launch": kbytes[dom]}
    stack_bytes = sum(decode_layer_bytes(wl, T, a) for a in n_active)
    replay = stack.last_replay_ms
    result = {
        "metric": METRIC, "value": T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "median_ms_per_step": replay["median"], "mean_ms_per_step": replay["mean"],
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "layers": args.layers, "tokens_per_step": T, "hidden": wl.H,
                   "experts": wl.E, "top_k": wl.k, "intermediate": wl.I, "weights": "Q8_0",
                   "activations": "fp32", "graph": "hip graph of the whole stack",
                   "calls_per_layer": {"layer": "moe_decode_layer", "two": "moe_route_permute + moe_expert_ffn",
                                       "four": "moe_route, moe_permute, moe_expert_ffn, moe_combine"}[args.calls]},
        "roofline": roofline,
        "stack_hbm_gbs": stack_bytes / (ms_per_step * 1e-3) / 1e9,
    }
    legs = set(args.legs.split(",")) if not args.no_extras else set()
    if args.no_cache:
        legs.discard("cache")
    if "batches" in legs:
        extra = {}
        for tb in wl.batches:
            if tb == T:
                continue
            _, bb, w2, _ = time_graph(stack, tb, max(10, args.steps // 2), args.warmup)
            ms2 = w2 * 1e3 / max(10, args.steps // 2)
            na2 = stack.n_active(bb)
            extra[str(tb)] = {"tokens_per_s": tb / (ms2 * 1e-3), "ms_per_step": ms2,
                              "median_ms_per_step": stack.last_replay_ms["median"],
                              "mean_active_experts": sum(na2) / len(na2),
                              "stack_hbm_gbs": sum(decode_layer_bytes(wl, tb, a) for a in na2) / (ms2 * 1e-3) / 1e9}
            log(f"T={tb}: {ms2:.3f} ms/step, {tb / (ms2 * 1e-3):.1f} tok/s")
        result["batches"] = extra
    del stack
    torch.cuda.empty_cache()
    if "wide" in legs:
        try:
            result["wide"] = wide_extra(ctx)
        except Exception as e:  # reported, never silently dropped
            result["wide"] = {"error": repr(e)}
    if "prefill" in legs:
        try:
            result["prefill"] = prefill_extra(ctx)
            log(f"prefill: {result['prefill']['tokens_per_s']:.0f} tok/s, FFN "
                f"{result['prefill']['ffn_tflops']:.1f} TFLOP/s")
        except Exception as e:  # reported, never silently dropped
            result["prefill"] = {"error": repr(e)}
    if "prefill_stream" in legs:
        try:
            result["prefill_stream"] = prefill_stream_extra(ctx)
            ps = result["prefill_stream"]
            log(f"prefill streamed: {ps['ms_per_layer']:.2f} ms/layer ({ps['tokens_per_s']:.0f} tok/s), H2D "
                f"{ps['h2d_gbs']:.1f} GB/s; copy alone {ps['copy_only_ms_per_layer']:.2f}, compute alone "
                f"{ps['compute_only_ms_per_layer']:.2f}, serial {ps['serial_ms_per_layer']:.2f} ms/layer; overlap "
                f"efficiency {ps['overlap_efficiency']:.2f}")
        except Exception as e:
            result["prefill_stream"] = {"error": repr(e)}
    if "block_types" in legs:
        try:
            result["block_types"] = types_extra(ctx)
        except Exception as e:
            result["block_types"] = {"error": repr(e)}
    if "cache" in legs:
        try:
            result["cache"] = cache_extra(ctx, steps=args.cache_steps, sweep_steps=args.sweep_steps)
            c = result["cache"]
            log(f"cache: {c['tokens_per_s']:.1f} tok/s, hit rate {c['hit_rate']:.3f}, warm "
                f"{c['warm']['tokens_per_s']:.1f} tok/s at {c['warm']['hit_rate']:.3f}, "
                f"H2D {c['h2d_gbs']:.1f} GB/s of {c['h2d_copy_ceiling_gbs']:.1f}")
        except Exception as e:
            result["cache"] = {"error": repr(e)}
    cache_misses = result.get("cache", {}).pop("_misses_per_layer", None)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        cb = cpu_baselines(cache_misses)
        head = cb.get(f"decode_q8_0_h2048_e128 T={T}", cb["decode_q8_0_h2048_e128 T=1"])
        result["cpu_baseline"] = {
            "value": head["tokens_per_s_stack"], "unit": "tokens/s", "cores": cb["cores"], "kind": "oracle",
            "cpu_model": cb["cpu_model"],
            "sample": f"NumPy float64 oracle, {head['layer_forwards']} layer forwards of the 48-layer stack "
                      f"(one per layer) run concurrently on {cb['cores']} threads in {head['seconds']:.1f}s, "
                      f"scaled to the stack; experts are 16 generated ones repeated over the ids"}
        result["cpu_baselines"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
