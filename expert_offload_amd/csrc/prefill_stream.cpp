// Layer streaming for prefill: the experts of every layer live in pinned
// host memory and pass through two device buffers of one layer each.
//
// A long prompt touches nearly every expert of every layer, so a cache buys
// little there; instead the next layer's experts are copied over PCIe while
// the current layer computes ("FreeToken Inference Engine: 3x Speed Boost
// for MoE Models", section "Dual-Buffering to Solve the Prefill
// Bottleneck").
//
// Per call for layer l: if no buffer holds l, it is copied now into the
// buffer the previous layer did not use (demand load).  The routing runs on
// the compute stream at once (it needs no expert bytes), then the FFN and
// the combine run out of that buffer once l's copy has landed, and a
// done-event marks the buffer free.  Then layer l+1 is copied into the
// other buffer, after the layer that last read that buffer has finished.
//
// The copies are HSA asynchronous copies (the DMA engines, with one
// completion signal per buffer), waited for on the host: they put no packet
// into any HIP queue, so the copy and the compute overlap however HIP maps
// streams onto hardware queues (two streams that share one queue run their
// work in order).  The cost is that a call returns only once its layer's
// copy has landed and the next layer's copy has been issued, i.e. after
// the previous layer's FFN.  Without the HSA runtime, or with
// MOE_STREAM_HIP_COPY set in the environment at create time, the copies are
// hipMemcpyAsync calls on the caller's copy stream ordered by events.
#include <cstdlib>
#include <vector>

#include "hsa_copy.h"
#include "moe_internal.h"

using namespace moe;

struct moe_prefill_stream {
  int device = 0;
  int L = 0, E = 0, qtype = 0, H = 0, I = 0;
  size_t slot_bytes = 0, layer_bytes = 0;
  uint8_t* d_bufs = nullptr;        // caller-owned: 2 buffers of E slots
  const uint8_t* h_pool = nullptr;  // caller-owned pinned [L][E] slots
  int32_t* d_ident = nullptr;       // slot of expert e in a buffer: e
  int buf_layer[2] = {-1, -1};      // layer held (or being copied) per buffer
  bool copied[2] = {false, false}, used[2] = {false, false};
  hipEvent_t copy_ev[2] = {}, done_ev[2] = {};
  int last_buf = -1;
  int64_t loads = 0, demand_loads = 0;
  bool hsa_ok = false;  // copies through the HSA runtime
  hsa_agent_t hsa_gpu{}, hsa_cpu{};
  hsa_signal_t sig[2] = {};  // 1 while a copy into the buffer is in flight
};

static void sig_wait(const moe_prefill_stream* s, int b) {
  while (hsa_signal_wait_scacquire(s->sig[b], HSA_SIGNAL_CONDITION_EQ, 0, UINT64_MAX, HSA_WAIT_STATE_BLOCKED) != 0) {
  }
}

static void hsa_setup(moe_prefill_stream* s) {
  const char* env = std::getenv("MOE_STREAM_HIP_COPY");
  if (env && *env && *env != '0') return;
  if (hsa_init() != HSA_STATUS_SUCCESS) return;
  if (!hsa_agents_of(s->device, &s->hsa_gpu, &s->hsa_cpu)) {
    hsa_shut_down();
    return;
  }
  if (hsa_signal_create(0, 0, nullptr, &s->sig[0]) != HSA_STATUS_SUCCESS) {
    hsa_shut_down();
    return;
  }
  if (hsa_signal_create(0, 0, nullptr, &s->sig[1]) != HSA_STATUS_SUCCESS) {
    hsa_signal_destroy(s->sig[0]);
    hsa_shut_down();
    return;
  }
  s->hsa_ok = true;
}

static int load_layer_hsa(moe_prefill_stream* s, int b, int layer) {
  hipError_t e;
  // after the last reader of the buffer and after an earlier copy into it
  if (s->used[b] && (e = hipEventSynchronize(s->done_ev[b])) != hipSuccess)
    return hip_error(e, "hipEventSynchronize(buffer free)");
  sig_wait(s, b);
  hsa_signal_store_screlease(s->sig[b], 1);
  const hsa_status_t st =
      hsa_amd_memory_async_copy(s->d_bufs + (size_t)b * s->layer_bytes, s->hsa_gpu,
                                s->h_pool + (size_t)layer * s->layer_bytes, s->hsa_cpu, s->layer_bytes, 0, nullptr,
                                s->sig[b]);
  if (st != HSA_STATUS_SUCCESS) {
    hsa_signal_store_screlease(s->sig[b], 0);
    s->buf_layer[b] = -1;
    return set_error(MOE_ERR_HIP, "hsa_amd_memory_async_copy(layer experts) failed (status %d)", (int)st);
  }
  s->buf_layer[b] = layer;
  ++s->loads;
  return MOE_OK;
}

static int load_layer(moe_prefill_stream* s, int b, int layer, hipStream_t cs) {
  if (s->hsa_ok) return load_layer_hsa(s, b, layer);
  hipError_t e;
  // after the last reader of the buffer, and after an earlier copy into it
  // that may sit on another copy stream
  if (s->used[b] && (e = hipStreamWaitEvent(cs, s->done_ev[b], 0)) != hipSuccess)
    return hip_error(e, "hipStreamWaitEvent(buffer free)");
  if (s->copied[b] && (e = hipStreamWaitEvent(cs, s->copy_ev[b], 0)) != hipSuccess)
    return hip_error(e, "hipStreamWaitEvent(earlier copy)");
  if ((e = hipMemcpyAsync(s->d_bufs + (size_t)b * s->layer_bytes, s->h_pool + (size_t)layer * s->layer_bytes,
                          s->layer_bytes, hipMemcpyHostToDevice, cs)) != hipSuccess)
    return hip_error(e, "hipMemcpyAsync(layer experts)");
  if ((e = hipEventRecord(s->copy_ev[b], cs)) != hipSuccess) return hip_error(e, "hipEventRecord(copy)");
  s->buf_layer[b] = layer;
  s->copied[b] = true;
  ++s->loads;
  return MOE_OK;
}

extern "C" {

int prefill_stream_destroy(moe_prefill_stream* s);

int prefill_stream_create(int L, int E, int qtype, int H, int I, void* d_bufs, const void* h_pool,
                          moe_prefill_stream** out) {
  clear_error();
  if (!out) return set_error(MOE_ERR_INVALID_ARG, "prefill_stream_create: out is NULL");
  if (!qtype_supported(qtype))
    return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "prefill_stream_create: block type %d is not supported", qtype);
  if (L < 1 || E < 1 || E > kMaxE)
    return set_error(MOE_ERR_INVALID_ARG, "prefill_stream_create: L=%d E=%d", L, E);
  if (H <= 0 || I <= 0 || H % kGroupWeights || I % kGroupWeights)
    return set_error(MOE_ERR_INVALID_ARG, "prefill_stream_create: H=%d I=%d must be multiples of %d", H, I,
                     kGroupWeights);
  if (!d_bufs || !h_pool) return set_error(MOE_ERR_INVALID_ARG, "prefill_stream_create: NULL buffer or pool");
  if (!aligned(d_bufs, 16)) return set_error(MOE_ERR_ALIGNMENT, "prefill_stream_create: d_bufs not 16-byte aligned");
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, h_pool);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return set_error(MOE_ERR_NOT_PINNED,
                     "prefill_stream_create: the host expert pool is not pinned (allocate it with hipHostMalloc)");
  }
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_error(e, "hipGetDevice");
  moe_prefill_stream* s = new moe_prefill_stream;
  s->device = dev;
  s->L = L; s->E = E; s->qtype = qtype; s->H = H; s->I = I;
  s->slot_bytes = slot_bytes_of(qtype, H, I);
  s->layer_bytes = s->slot_bytes * (size_t)E;
  s->d_bufs = (uint8_t*)d_bufs;
  s->h_pool = (const uint8_t*)h_pool;
  std::vector<int32_t> ident(E);
  for (int i = 0; i < E; ++i) ident[i] = i;
  if ((e = hipMalloc(&s->d_ident, sizeof(int32_t) * E)) != hipSuccess ||
      (e = hipMemcpy(s->d_ident, ident.data(), sizeof(int32_t) * E, hipMemcpyHostToDevice)) != hipSuccess) {
    prefill_stream_destroy(s);
    return hip_error(e, "prefill_stream_create: identity slot table");
  }
  for (int b = 0; b < 2; ++b) {
    if ((e = hipEventCreateWithFlags(&s->copy_ev[b], hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&s->done_ev[b], hipEventDisableTiming)) != hipSuccess) {
      prefill_stream_destroy(s);
      return hip_error(e, "hipEventCreate");
    }
  }
  hsa_setup(s);
  *out = s;
  return MOE_OK;
}

int prefill_stream_destroy(moe_prefill_stream* s) {
  clear_error();
  if (!s) return MOE_OK;
  (void)hipDeviceSynchronize();
  if (s->hsa_ok) {
    for (int b = 0; b < 2; ++b) {
      sig_wait(s, b);
      hsa_signal_destroy(s->sig[b]);
    }
    hsa_shut_down();
  }
  for (int b = 0; b < 2; ++b) {
    if (s->copy_ev[b]) (void)hipEventDestroy(s->copy_ev[b]);
    if (s->done_ev[b]) (void)hipEventDestroy(s->done_ev[b]);
  }
  if (s->d_ident) (void)hipFree(s->d_ident);
  delete s;
  return MOE_OK;
}

int prefill_stream_stats(moe_prefill_stream* s, int64_t* loads, int64_t* demand_loads) {
  clear_error();
  if (!s) return set_error(MOE_ERR_INVALID_ARG, "prefill_stream_stats: stream is NULL");
  if (loads) *loads = s->loads;
  if (demand_loads) *demand_loads = s->demand_loads;
  return MOE_OK;
}

int prefill_stream_layer(moe_prefill_stream* s, moe_ctx* ctx, int layer, const moe_ffn_args* args,
                         const float* router_w, const float* bias, const float* logits_in, float* logits_out,
                         int32_t* topk_ids, int32_t* pair_pos, void* route_ws, size_t route_ws_bytes,
                         void* copy_stream, void* compute_stream) {
  clear_error();
  if (!s || !ctx || !args) return set_error(MOE_ERR_INVALID_ARG, "prefill_stream_layer: stream, ctx or args is NULL");
  if (layer < 0 || layer >= s->L)
    return set_error(MOE_ERR_INVALID_ARG, "prefill_stream_layer: layer %d not in [0, %d)", layer, s->L);
  if (args->H != s->H || args->I != s->I || args->E != s->E || args->qtype != s->qtype)
    return set_error(MOE_ERR_INVALID_ARG,
                     "prefill_stream_layer: args H=%d I=%d E=%d qtype=%d differ from the stream's H=%d I=%d E=%d "
                     "qtype=%d",
                     args->H, args->I, args->E, args->qtype, s->H, s->I, s->E, s->qtype);
  if (!args->topk_w || !args->out)
    return set_error(MOE_ERR_INVALID_ARG, "prefill_stream_layer: args.topk_w and args.out are required");
  if (args->expert_mask)
    return set_error(MOE_ERR_INVALID_ARG, "prefill_stream_layer: args.expert_mask must be NULL (every expert runs)");
  if (args->T == 0) return MOE_OK;
  hipError_t e = hipSetDevice(s->device);
  if (e != hipSuccess) return hip_error(e, "hipSetDevice");
  hipStream_t cs = (hipStream_t)copy_stream, ks = (hipStream_t)compute_stream;
  int rc;
  int b = s->buf_layer[0] == layer ? 0 : s->buf_layer[1] == layer ? 1 : -1;
  if (b < 0) {
    b = s->last_buf < 0 ? 0 : 1 - s->last_buf;
    if ((rc = load_layer(s, b, layer, cs))) return rc;
    ++s->demand_loads;
  }
  // the routing needs no expert bytes: it runs while the copy is in flight
  rc = moe_route_permute(ctx, args->x, args->x_dtype, router_w, bias, logits_in, args->T, s->H, s->E, args->k,
                         logits_out, topk_ids, const_cast<float*>(args->topk_w),
                         const_cast<int32_t*>(args->expert_offsets), const_cast<int32_t*>(args->sorted_pairs),
                         pair_pos, const_cast<int32_t*>(args->active), route_ws, route_ws_bytes, compute_stream);
  if (rc) return rc;
  if (s->hsa_ok)
    sig_wait(s, b);
  else if ((e = hipStreamWaitEvent(ks, s->copy_ev[b], 0)) != hipSuccess)
    return hip_error(e, "hipStreamWaitEvent(copy)");
  moe_ffn_args a = *args;
  a.pool_base = s->d_bufs + (size_t)b * s->layer_bytes;
  a.slot_bytes = s->slot_bytes;
  a.n_slots = s->E;
  a.slot_table = s->d_ident;
  if ((rc = moe_expert_ffn(ctx, &a, compute_stream))) return rc;
  if ((e = hipEventRecord(s->done_ev[b], ks)) != hipSuccess) return hip_error(e, "hipEventRecord(layer done)");
  s->used[b] = true;
  s->last_buf = b;
  // dual buffering: the next layer's experts cross PCIe while this one computes
  const int next = layer + 1;
  if (next < s->L && s->buf_layer[1 - b] != next) {
    if ((rc = load_layer(s, 1 - b, next, cs))) return rc;
  }
  return MOE_OK;
}

}  // extern "C"
