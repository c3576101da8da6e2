// Router: logits, softmax, top-k (ties to the lower expert id) and
// renormalisation of the kept probabilities.
//
// Each token activates only a few experts ("FreeToken github moe: Setup
// Guide & MoE Runtime Comparison", introduction); the selection rule is the
// usual softmax -> top-k -> renormalise of routed MoE layers.
#include <cfloat>
#include <climits>

#include "device_common.h"

namespace moe {

// logits[t][e] = sum_h x[t][h] * Wr[e][h] (+ bias[e]).  One wave per expert;
// the wave strides over h with 4-wide loads, then reduces.
template <typename XT>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ bias, int T,
                                                            int H, int E, float* __restrict__ logits) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const float* w = wr + (size_t)e * H;
  const float b = bias ? bias[e] : 0.0f;
  for (int t = 0; t < T; ++t) {
    const XT* xt = x + (size_t)t * H;
    float acc = 0.0f;
    for (int h = lane * 4; h < H; h += 4 * kWave) {
      const float4 wv = *reinterpret_cast<const float4*>(w + h);
      float xv[4];
      if constexpr (sizeof(XT) == 4) {
        const float4 v = *reinterpret_cast<const float4*>(xt + h);
        xv[0] = v.x; xv[1] = v.y; xv[2] = v.z; xv[3] = v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(xt + h);
        xv[0] = bf16_to_f32(v.x & 0xFFFF); xv[1] = bf16_to_f32(v.x >> 16);
        xv[2] = bf16_to_f32(v.y & 0xFFFF); xv[3] = bf16_to_f32(v.y >> 16);
      }
      acc = fmaf(xv[0], wv.x, acc);
      acc = fmaf(xv[1], wv.y, acc);
      acc = fmaf(xv[2], wv.z, acc);
      acc = fmaf(xv[3], wv.w, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) logits[(size_t)t * E + e] = acc + b;
  }
}

// One wave per token: k rounds of a wave-wide argmax over the fp32 logits
// (larger value wins, equal values go to the lower id), then
// w_j = exp(l_j - l_max) / sum_j' exp(l_j' - l_max) over the kept experts,
// which equals the softmax probabilities renormalised over the top k.
// NaN logits are treated as -inf.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ src,
                                                   const float* __restrict__ bias, int T, int E,
                                                   int k, float* __restrict__ logits_out,
                                                   int32_t* __restrict__ ids, float* __restrict__ w) {
  constexpr int kPer = kMaxE / kWave;  // 16 logits per lane at E = 1024
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + kWave * i;
    float val = -INFINITY;
    if (e < E) {
      val = src[(size_t)t * E + e];
      if (bias) val += bias[e];
      if (logits_out) logits_out[(size_t)t * E + e] = val;
      if (val != val) val = -INFINITY;
    }
    v[i] = val;
  }
  unsigned taken = 0;
  float my_val = -INFINITY;
  for (int j = 0; j < k; ++j) {
    float best = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > best || (v[i] == best && e < bi))) {
        best = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ob = __shfl_xor(best, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    if (lane == (bi & (kWave - 1))) taken |= 1u << (bi / kWave);
    if (lane == j) my_val = best;
    if (lane == 0) ids[(size_t)t * k + j] = bi;
  }
  const float m = __shfl(my_val, 0, kWave);
  const float ex = lane < k ? expf(my_val - m) : 0.0f;
  const float s = wave_sum(ex);
  if (lane < k) w[(size_t)t * k + lane] = ex / s;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_route(moe_ctx* ctx, const void* x, int x_dtype, const float* router_w,
                         const float* bias, const float* logits_in, int T, int H, int E, int k,
                         float* logits_out, int32_t* topk_ids, float* topk_w, void* stream) {
  clear_error();
  if (!ctx) return set_error(MOE_ERR_INVALID_ARG, "moe_route: ctx is NULL");
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E || k > kMaxK)
    return set_error(MOE_ERR_INVALID_ARG, "moe_route: need T >= 0, 1 <= k <= E <= %d, k <= %d (T=%d E=%d k=%d)",
                     kMaxE, kMaxK, T, E, k);
  if (T == 0) return MOE_OK;
  if (!topk_ids || !topk_w) return set_error(MOE_ERR_INVALID_ARG, "moe_route: topk_ids/topk_w is NULL");
  if (!logits_in) {
    if (!x || !router_w)
      return set_error(MOE_ERR_INVALID_ARG, "moe_route: x and router_w are required without logits_in");
    if (!logits_out)
      return set_error(MOE_ERR_INVALID_ARG, "moe_route: logits_out is required when logits are computed");
    if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16)
      return set_error(MOE_ERR_INVALID_ARG, "moe_route: x_dtype %d unknown", x_dtype);
    if (H <= 0 || H % 256)
      return set_error(MOE_ERR_INVALID_ARG, "moe_route: H=%d must be a positive multiple of 256", H);
    if (!aligned(x, 16) || !aligned(router_w, 16))
      return set_error(MOE_ERR_ALIGNMENT, "moe_route: x and router_w must be 16-byte aligned");
  }
  int rc = ensure_device(ctx);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const float* src = logits_in;
  const float* tk_bias = bias;
  if (!logits_in) {
    dim3 grid((E + 3) / 4);
    if (x_dtype == MOE_DTYPE_F32)
      router_logits_kernel<float><<<grid, 256, 0, s>>>((const float*)x, router_w, bias, T, H, E, logits_out);
    else
      router_logits_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)x, router_w, bias, T, H, E,
                                                          logits_out);
    if ((rc = check_launch("router_logits_kernel"))) return rc;
    src = logits_out;
    tk_bias = nullptr;
  }
  topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(src, tk_bias, T, E, k, logits_in ? logits_out : nullptr,
                                          topk_ids, topk_w);
  return check_launch("topk_kernel");
}
