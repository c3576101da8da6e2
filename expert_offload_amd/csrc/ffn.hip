// moe_expert_ffn: validation and dispatch of the expert-FFN kernels.
#include <algorithm>

#include "ffn.h"

namespace moe {

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace: decode keeps h as T*k x I fp32 in grouped (sorted) pair order;
// prefill keeps a tile list and h as bf16.  One size covers both.  The
// int8-activation decode adds, after h, the codes, scales and code sums of
// x and of h (256-byte aligned regions).
struct Q8aLayout {
  size_t xq, xs, xsum, hq, hs, hsum, end;
};
static Q8aLayout q8a_layout(const moe_ffn_args* a) {
  const size_t P = (size_t)a->T * a->k, xb = (size_t)a->T * a->H / kQK, hb = P * a->I / kQK;
  Q8aLayout l;
  l.xq = align_up(P * a->I * sizeof(float), 256);
  l.xs = align_up(l.xq + (size_t)a->T * a->H, 256);
  l.xsum = align_up(l.xs + xb * sizeof(float), 256);
  l.hq = align_up(l.xsum + xb * sizeof(int), 256);
  l.hs = align_up(l.hq + P * a->I, 256);
  l.hsum = align_up(l.hs + hb * sizeof(float), 256);
  l.end = align_up(l.hsum + hb * sizeof(int), 256);
  return l;
}
static size_t ffn_ws_bytes(const moe_ffn_args* a) {
  if (a->mode == MOE_MODE_DECODE_Q8A) return q8a_layout(a).end;
  const size_t dec = align_up((size_t)a->T * a->k * a->I * sizeof(float), 256);
  const size_t pre = align_up(prefill_ws_bytes(a->T, a->k, a->I, a->E), 256);
  return dec > pre ? dec : pre;
}

static int validate_ffn(const moe_ffn_args* a, bool need_buffers) {
  if (!a) return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: args is NULL");
  if (!qtype_supported(a->qtype))
    return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "moe_expert_ffn: block type %d is not supported", a->qtype);
  if (a->H <= 0 || a->I <= 0 || a->H % kGroupWeights || a->I % kGroupWeights)
    return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: H=%d and I=%d must be positive multiples of %d",
                     a->H, a->I, kGroupWeights);
  if (a->T < 0 || a->E < 1 || a->E > kMaxE || a->k < 1 || a->k > a->E)
    return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: need T >= 0, 1 <= k <= E <= %d (T=%d k=%d E=%d)",
                     kMaxE, a->T, a->k, a->E);
  if (a->mode != MOE_MODE_DECODE && a->mode != MOE_MODE_PREFILL && a->mode != MOE_MODE_DECODE_Q8A)
    return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: mode %d unknown", a->mode);
  if (a->x_dtype != MOE_DTYPE_F32 && a->x_dtype != MOE_DTYPE_BF16)
    return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: x_dtype %d unknown", a->x_dtype);
  if (a->mode != MOE_MODE_PREFILL && a->x_dtype != MOE_DTYPE_F32)
    return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: decode modes take fp32 activations");
  if (a->mode == MOE_MODE_DECODE_Q8A) {
    if (a->qtype != MOE_QTYPE_Q4_0 && a->qtype != MOE_QTYPE_Q8_0)
      return set_error(MOE_ERR_UNSUPPORTED_QTYPE,
                       "moe_expert_ffn: int8-activation decode takes Q4_0 and Q8_0 banks, not %s (type %d)",
                       qtype_name(a->qtype), a->qtype);
    if (!decode_gemv_supported(a->H, a->I, a->T, a->k))
      return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: int8-activation decode needs T*k <= 1024 (T=%d k=%d)",
                       a->T, a->k);
  }
  if (a->slot_bytes < slot_bytes_of(a->qtype, a->H, a->I))
    return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: slot_bytes %zu below one %s expert (%zu)",
                     a->slot_bytes, qtype_name(a->qtype), slot_bytes_of(a->qtype, a->H, a->I));
  if (a->n_slots < 1) return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: n_slots=%d", a->n_slots);
  if (a->slot_bytes % 16)
    return set_error(MOE_ERR_ALIGNMENT, "moe_expert_ffn: slot_bytes must be a multiple of 16");
  if (!need_buffers || a->T == 0) return MOE_OK;
  if (!a->pool_base || !a->slot_table || !a->x || !a->expert_offsets || !a->sorted_pairs ||
      !a->active || !a->y_pairs)
    return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: NULL buffer in args");
  if (!aligned(a->pool_base, 16) || !aligned(a->x, 16) || !aligned(a->y_pairs, 16))
    return set_error(MOE_ERR_ALIGNMENT, "moe_expert_ffn: pool_base, x and y_pairs must be 16-byte aligned");
  if (a->ws_bytes < ffn_ws_bytes(a) || (ffn_ws_bytes(a) && !a->ws))
    return set_error(MOE_ERR_WORKSPACE, "moe_expert_ffn: workspace holds %zu bytes, needs %zu",
                     a->ws_bytes, ffn_ws_bytes(a));
  if (!aligned(a->ws, 256)) return set_error(MOE_ERR_ALIGNMENT, "moe_expert_ffn: ws must be 256-byte aligned");
  if (a->out) {
    if (!a->topk_w) return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: out needs topk_w");
    if (a->expert_mask)
      return set_error(MOE_ERR_INVALID_ARG,
                       "moe_expert_ffn: the fused combine (out) needs every expert in one call (no expert_mask)");
    if (!aligned(a->out, 16)) return set_error(MOE_ERR_ALIGNMENT, "moe_expert_ffn: out must be 16-byte aligned");
  }
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_expert_ffn_workspace_size(const moe_ffn_args* args, size_t* bytes) {
  clear_error();
  int rc = validate_ffn(args, false);
  if (rc) return rc;
  if (!bytes) return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn_workspace_size: bytes is NULL");
  *bytes = ffn_ws_bytes(args);
  return MOE_OK;
}

static FfnParams ffn_params(const moe_ctx* ctx, const moe_ffn_args* a) {
  FfnParams p;
  p.pool = (const uint8_t*)a->pool_base;
  p.slot_bytes = a->slot_bytes;
  p.n_slots = a->n_slots;
  p.qtype = a->qtype;
  p.H = a->H; p.I = a->I; p.T = a->T; p.k = a->k; p.E = a->E;
  p.slot_table = a->slot_table;
  p.offsets = a->expert_offsets;
  p.sorted_pairs = a->sorted_pairs;
  p.active = a->active;
  p.mask = a->expert_mask;
  p.y = a->y_pairs;
  p.hbuf = (float*)a->ws;
  p.err = ctx->d_err;
  p.topk_w = a->topk_w;
  p.out = a->out;
  p.xq = p.hq = nullptr;
  p.xs = p.hs = nullptr;
  p.xsum = p.hsum = nullptr;
  if (a->mode == MOE_MODE_DECODE_Q8A) {
    const Q8aLayout l = q8a_layout(a);
    char* ws = (char*)a->ws;
    p.xq = (int8_t*)(ws + l.xq);
    p.xs = (float*)(ws + l.xs);
    p.xsum = (int*)(ws + l.xsum);
    p.hq = (int8_t*)(ws + l.hq);
    p.hs = (float*)(ws + l.hs);
    p.hsum = (int*)(ws + l.hsum);
  }
  return p;
}

extern "C" int moe_expert_ffn(moe_ctx* ctx, const moe_ffn_args* a, void* stream) {
  clear_error();
  if (!ctx) return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: ctx is NULL");
  int rc = validate_ffn(a, true);
  if (rc) return rc;
  if (a->T == 0) return MOE_OK;
  if ((rc = ensure_device(ctx))) return rc;
  FfnParams p = ffn_params(ctx, a);
  hipStream_t s = (hipStream_t)stream;
  if (a->mode == MOE_MODE_DECODE_Q8A || (a->mode == MOE_MODE_DECODE && decode_gemv_supported(a->H, a->I, a->T, a->k)))
    return launch_ffn_decode(ctx, p, (const float*)a->x, s);
  p.out = nullptr;
  if (a->mode == MOE_MODE_PREFILL && a->x_dtype == MOE_DTYPE_BF16 && prefill_mfma_supported(a->H, a->I))
    rc = launch_ffn_prefill(ctx, p, a->x, a->ws, s);
  else
    rc = launch_ffn_valu(ctx, p, a->x, a->x_dtype, s);
  if (rc || !a->out) return rc;
  return launch_combine(ctx, a->y_pairs, a->topk_w, a->T, a->k, a->H, a->out, s);
}

extern "C" int moe_decode_layer(moe_ctx* ctx, const moe_ffn_args* a, const float* router_w, const float* bias,
                                const float* logits_in, float* logits_out, int32_t* topk_ids, int32_t* pair_pos,
                                void* stream) {
  clear_error();
  if (!ctx || !a) return set_error(MOE_ERR_INVALID_ARG, "moe_decode_layer: ctx or args is NULL");
  if (a->mode != MOE_MODE_DECODE && a->mode != MOE_MODE_DECODE_Q8A)
    return set_error(MOE_ERR_INVALID_ARG, "moe_decode_layer: args.mode must be MOE_MODE_DECODE or _DECODE_Q8A");
  if (!a->topk_w || !a->out)
    return set_error(MOE_ERR_INVALID_ARG, "moe_decode_layer: args.topk_w and args.out are required");
  if (a->expert_mask) return set_error(MOE_ERR_INVALID_ARG, "moe_decode_layer: args.expert_mask must be NULL");
  // the routing results go to the args' topk_w / expert_offsets /
  // sorted_pairs / active buffers, which moe_expert_ffn only reads
  float* topk_w = const_cast<float*>(a->topk_w);
  int32_t* offsets = const_cast<int32_t*>(a->expert_offsets);
  int32_t* sorted = const_cast<int32_t*>(a->sorted_pairs);
  int32_t* active = const_cast<int32_t*>(a->active);
  int rc = validate_route_args("moe_decode_layer", a->x, a->x_dtype, router_w, logits_in, a->T, a->H, a->E, a->k,
                               logits_out, topk_ids, topk_w);
  if (rc) return rc;
  if ((rc = validate_ffn(a, true))) return rc;
  if (a->T == 0) return MOE_OK;
  if (!pair_pos) return set_error(MOE_ERR_INVALID_ARG, "moe_decode_layer: pair_pos is NULL");
  if ((rc = ensure_device(ctx))) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (a->mode == MOE_MODE_DECODE_Q8A || !decode_route_supported(a->H, a->I, a->T, a->k)) {
    rc = moe_route_permute(ctx, a->x, a->x_dtype, router_w, bias, logits_in, a->T, a->H, a->E, a->k, logits_out,
                           topk_ids, topk_w, offsets, sorted, pair_pos, active, nullptr, 0, stream);
    if (rc) return rc;
    return moe_expert_ffn(ctx, a, stream);
  }
  RouteArgs ra{};
  if (!logits_in) {
    if ((rc = launch_router_logits(ctx, a->x, a->x_dtype, router_w, bias, a->T, a->H, a->E, logits_out, s)))
      return rc;
    ra.logits = logits_out;  // biased already
  } else {
    ra.logits = logits_in;
    ra.bias = bias;
    ra.logits_out = logits_out;
  }
  ra.ids = topk_ids;
  ra.w = topk_w;
  ra.offsets = offsets;
  ra.sorted_pairs = sorted;
  ra.pair_pos = pair_pos;
  ra.active = active;
  return launch_ffn_decode(ctx, ffn_params(ctx, a), (const float*)a->x, s, &ra);
}
