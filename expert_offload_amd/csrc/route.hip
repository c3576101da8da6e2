// Router: logits, softmax, top-k (ties to the lower expert id) and
// renormalisation of the kept probabilities; plus the fused decode variant
// that also groups the pairs by expert in the same launch.
//
// Each token activates only a few experts ("FreeToken github moe: Setup
// Guide & MoE Runtime Comparison", introduction); the selection rule is the
// usual softmax -> top-k -> renormalise of routed MoE layers.
#include <cfloat>
#include <climits>

#include "ffn.h"
#include "route_common.h"

namespace moe {

int launch_permute(moe_ctx* ctx, const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pairs,
                   int32_t* pair_pos, int32_t* active, void* ws, size_t ws_bytes, hipStream_t s);
size_t permute_ws_bytes(long long P, int E);

// One workgroup per EPB experts and chunk of kRouterChunk tokens: its four
// wavefronts each take a quarter of the hidden dimension, partial sums meet
// in LDS.  TB tokens at a time: their activation loads go out together and
// serve the EPB experts' dot products side by side.  Each (token, expert)
// sum keeps one fixed order (a lane's FMAs in h order, the wavefront's DPP
// tree, the quarters in pairs), so neither TB, EPB nor the chunking changes
// a logit; with fewer than TB tokens left the last one is repeated and the
// repeats are dropped.  The chunks run in parallel workgroups, and EPB > 1
// reads each token row once per EPB experts rather than once per expert (a
// 64-token batch of 512 experts otherwise re-reads 268 MB of activations):
// that batch's logits took 19.5 us with one workgroup per expert, 14.6 us
// with 16-token chunks and 13.5 us with four experts per workgroup.
constexpr int kRouterChunk = 16;
template <typename XT, int TB, int EPB>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ bias, int T,
                                                            int H, int E, float* __restrict__ logits) {
  __shared__ float part[4][EPB][kRouterChunk];
  const int e0 = blockIdx.x * EPB;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int q = H / 4;  // H % 256 == 0, so q % 64 == 0
  const float* w[EPB];
#pragma unroll
  for (int i = 0; i < EPB; ++i) w[i] = wr + (size_t)min(e0 + i, E - 1) * H + wave * q;
  const int t0 = blockIdx.y * kRouterChunk;
  const int nt = min(kRouterChunk, T - t0);
  for (int tb = 0; tb < nt; tb += TB) {
    const XT* xt[TB];
#pragma unroll
    for (int u = 0; u < TB; ++u) xt[u] = x + (size_t)(t0 + min(tb + u, nt - 1)) * H + wave * q;
    float acc[EPB][TB];
#pragma unroll
    for (int i = 0; i < EPB; ++i)
#pragma unroll
      for (int u = 0; u < TB; ++u) acc[i][u] = 0.0f;
#pragma unroll 2
    for (int h = lane * 4; h < q; h += 4 * kWave) {
      float4 wv[EPB];
#pragma unroll
      for (int i = 0; i < EPB; ++i) wv[i] = *reinterpret_cast<const float4*>(w[i] + h);
      float xv[TB][4];
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        if constexpr (sizeof(XT) == 4) {
          const float4 v = *reinterpret_cast<const float4*>(xt[u] + h);
          xv[u][0] = v.x; xv[u][1] = v.y; xv[u][2] = v.z; xv[u][3] = v.w;
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(xt[u] + h);
          xv[u][0] = bf16_to_f32(v.x & 0xFFFF); xv[u][1] = bf16_to_f32(v.x >> 16);
          xv[u][2] = bf16_to_f32(v.y & 0xFFFF); xv[u][3] = bf16_to_f32(v.y >> 16);
        }
      }
#pragma unroll
      for (int i = 0; i < EPB; ++i)
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          acc[i][u] = fmaf(xv[u][0], wv[i].x, acc[i][u]);
          acc[i][u] = fmaf(xv[u][1], wv[i].y, acc[i][u]);
          acc[i][u] = fmaf(xv[u][2], wv[i].z, acc[i][u]);
          acc[i][u] = fmaf(xv[u][3], wv[i].w, acc[i][u]);
        }
    }
#pragma unroll
    for (int i = 0; i < EPB; ++i)
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const float v = wave_sum_dpp(acc[i][u]);
        if (lane == 0 && tb + u < nt) part[wave][i][tb + u] = v;
      }
  }
  __syncthreads();
  if (threadIdx.x < EPB * kRouterChunk) {
    const int i = threadIdx.x / kRouterChunk, u = threadIdx.x % kRouterChunk, e = e0 + i;
    if (u < nt && e < E) {
      const float b = bias ? bias[e] : 0.0f;
      logits[(size_t)(t0 + u) * E + e] = ((part[0][i][u] + part[1][i][u]) + (part[2][i][u] + part[3][i][u])) + b;
    }
  }
}

template <typename XT>
static void launch_router_logits_t(const XT* x, const float* router_w, const float* bias, int T, int H, int E,
                                   float* logits_out, hipStream_t s) {
  if (T <= 0) return;
  const unsigned chunks = (unsigned)((T + kRouterChunk - 1) / kRouterChunk);
  // four experts per workgroup once two chunks or more re-read the tokens
  constexpr int kEpb = 4;
  if (T > kRouterChunk)
    launch(router_logits_kernel<XT, 8, kEpb>, dim3((E + kEpb - 1) / kEpb, chunks), 256, 0, s, x, router_w, bias, T, H,
           E, logits_out);
  else if (T >= 8)
    launch(router_logits_kernel<XT, 8, 1>, dim3(E, chunks), 256, 0, s, x, router_w, bias, T, H, E, logits_out);
  else if (T >= 2)
    launch(router_logits_kernel<XT, 2, 1>, dim3(E, chunks), 256, 0, s, x, router_w, bias, T, H, E, logits_out);
  else
    launch(router_logits_kernel<XT, 1, 1>, dim3(E, chunks), 256, 0, s, x, router_w, bias, T, H, E, logits_out);
}

static void launch_router_logits_kernel(const void* x, int x_dtype, const float* router_w, const float* bias, int T,
                                        int H, int E, float* logits_out, hipStream_t s) {
  if (x_dtype == MOE_DTYPE_F32)
    launch_router_logits_t((const float*)x, router_w, bias, T, H, E, logits_out, s);
  else
    launch_router_logits_t((const uint16_t*)x, router_w, bias, T, H, E, logits_out, s);
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ src,
                                                   const float* __restrict__ bias, int T, int E,
                                                   int k, float* __restrict__ logits_out,
                                                   int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ TopkScratch sc[4];
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  wave_topk(src + (size_t)t * E, bias, E, k, logits_out ? logits_out + (size_t)t * E : nullptr,
            ids + (size_t)t * k, w + (size_t)t * k, nullptr, nullptr, nullptr, &sc[threadIdx.x >> 6]);
}

// Top-k of every token plus the stable grouping, in one workgroup (decode
// sized batches): removes a launch and keeps the ids in LDS between the two.
constexpr int kFusedMaxPairs = 4096;

constexpr int kTopkPermuteThreads = 512;
constexpr int kFusedMaxTokens = 2 * kTopkPermuteThreads / kWave;

struct TopkPermuteLds {
  int ids[kFusedMaxPairs];
  PermuteLds<kTopkPermuteThreads> perm;
};

__global__ __launch_bounds__(kTopkPermuteThreads) void topk_permute_kernel(
    const float* __restrict__ src, const float* __restrict__ bias, int T, int E, int k,
    float* __restrict__ logits_out, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ active, int* __restrict__ err, int32_t* __restrict__ ids_host, int32_t* ids_flag,
    int32_t seq) {
  __shared__ TopkPermuteLds s;
  __shared__ TopkScratch sc[kTopkPermuteThreads / kWave];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  constexpr int waves = kTopkPermuteThreads / kWave;
  for (int t = wave; t < T; t += waves)
    wave_topk(src + (size_t)t * E, bias, E, k, logits_out ? logits_out + (size_t)t * E : nullptr,
              ids + (size_t)t * k, w + (size_t)t * k, s.ids + t * k, nullptr, nullptr, &sc[wave]);
  __syncthreads();
  // a copy of the ids straight into host memory for a caller that waits for
  // them (the expert cache's lookup), instead of a separate read-back;
  static_assert(kTopkPermuteThreads >= 2 * kWave, "a second wavefront publishes the ids");
  if (ids_host && wave == 1) {
    // wavefront 1 publishes while wavefront 0 groups the pairs: every id
    // reaches host memory before the flag does, so a host that waits for
    // seq can start its lookup while this kernel still permutes.  Each
    // lane's system fence waits for the wavefront's outstanding stores (the
    // memory counter is per wavefront, so it covers all 64 lanes' stores);
    // the wave barrier keeps lane 0's flag store after every lane's fence
    // even if a later change lets lanes of this wavefront diverge.
    for (int i = lane; i < T * k; i += kWave) ids_host[i] = s.ids[i];
    __threadfence_system();
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) __hip_atomic_store(ids_flag, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  if (T * k <= 1024) {
    if (wave == 0) wave_permute(s.ids, T * k, E, offsets, sorted_pairs, pair_pos, active, err, s.perm.cnt, s.perm.cur);
  } else {
    block_permute<kTopkPermuteThreads>(s.ids, T * k, E, offsets, sorted_pairs, pair_pos, active, err, s.perm);
  }
}

int validate_route_args(const char* fn, const void* x, int x_dtype, const float* router_w,
                          const float* logits_in, int T, int H, int E, int k, float* logits_out,
                          int32_t* topk_ids, float* topk_w) {
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E || k > kMaxK)
    return set_error(MOE_ERR_INVALID_ARG, "%s: need T >= 0, 1 <= k <= E <= %d, k <= %d (T=%d E=%d k=%d)", fn,
                     kMaxE, kMaxK, T, E, k);
  if (T == 0) return MOE_OK;
  if (!topk_ids || !topk_w) return set_error(MOE_ERR_INVALID_ARG, "%s: topk_ids/topk_w is NULL", fn);
  if (!logits_in) {
    if (!x || !router_w)
      return set_error(MOE_ERR_INVALID_ARG, "%s: x and router_w are required without logits_in", fn);
    if (!logits_out)
      return set_error(MOE_ERR_INVALID_ARG, "%s: logits_out is required when logits are computed", fn);
    if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16)
      return set_error(MOE_ERR_INVALID_ARG, "%s: x_dtype %d unknown", fn, x_dtype);
    if (H <= 0 || H % 256)
      return set_error(MOE_ERR_INVALID_ARG, "%s: H=%d must be a positive multiple of 256", fn, H);
    if (!aligned(x, 16) || !aligned(router_w, 16))
      return set_error(MOE_ERR_ALIGNMENT, "%s: x and router_w must be 16-byte aligned", fn);
  }
  return MOE_OK;
}

int launch_router_logits(moe_ctx* ctx, const void* x, int x_dtype, const float* router_w, const float* bias, int T,
                         int H, int E, float* logits_out, hipStream_t s) {
  KernelTimer timer(ctx, "router_logits", s);
  launch_router_logits_kernel(x, x_dtype, router_w, bias, T, H, E, logits_out, s);
  return check_launch("router_logits_kernel");
}

static int launch_route(moe_ctx* ctx, const void* x, int x_dtype, const float* router_w, const float* bias,
                        const float* logits_in, int T, int H, int E, int k, float* logits_out,
                        int32_t* topk_ids, float* topk_w, hipStream_t s) {
  int rc;
  const float* src = logits_in;
  const float* tk_bias = bias;
  if (!logits_in) {
    {
      KernelTimer timer(ctx, "router_logits", s);
      launch_router_logits_kernel(x, x_dtype, router_w, bias, T, H, E, logits_out, s);
    }
    if ((rc = check_launch("router_logits_kernel"))) return rc;
    src = logits_out;
    tk_bias = nullptr;
  }
  KernelTimer timer(ctx, "topk", s);
  launch(topk_kernel, (T + 3) / 4, 256, 0, s, src, tk_bias, T, E, k, logits_in ? logits_out : nullptr, topk_ids,
                                          topk_w);
  return check_launch("topk_kernel");
}

}  // namespace moe

using namespace moe;

extern "C" int moe_route(moe_ctx* ctx, const void* x, int x_dtype, const float* router_w,
                         const float* bias, const float* logits_in, int T, int H, int E, int k,
                         float* logits_out, int32_t* topk_ids, float* topk_w, void* stream) {
  clear_error();
  if (!ctx) return set_error(MOE_ERR_INVALID_ARG, "moe_route: ctx is NULL");
  int rc = validate_route_args("moe_route", x, x_dtype, router_w, logits_in, T, H, E, k, logits_out, topk_ids, topk_w);
  if (rc || T == 0) return rc;
  if ((rc = ensure_device(ctx))) return rc;
  return launch_route(ctx, x, x_dtype, router_w, bias, logits_in, T, H, E, k, logits_out, topk_ids, topk_w,
                      (hipStream_t)stream);
}

extern "C" int moe_route_permute_workspace_size(int T, int k, int E, size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(MOE_ERR_INVALID_ARG, "moe_route_permute_workspace_size: bytes is NULL");
  if (T < 0 || k < 1 || E < 1 || E > kMaxE)
    return set_error(MOE_ERR_INVALID_ARG, "moe_route_permute_workspace_size: need T >= 0, k >= 1, 1 <= E <= %d",
                     kMaxE);
  // the separate permute of large batches takes its chunk counts from ws
  *bytes = (long long)T * k > kFusedMaxPairs ? permute_ws_bytes((long long)T * k, E) : 0;
  return MOE_OK;
}

extern "C" int moe_route_permute(moe_ctx* ctx, const void* x, int x_dtype, const float* router_w,
                                 const float* bias, const float* logits_in, int T, int H, int E, int k,
                                 float* logits_out, int32_t* topk_ids, float* topk_w,
                                 int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                                 int32_t* active, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  return route_permute_impl(ctx, x, x_dtype, router_w, bias, logits_in, T, H, E, k, logits_out, topk_ids, topk_w,
                            expert_offsets, sorted_pairs, pair_pos, active, ws, ws_bytes, nullptr, nullptr, 0, stream);
}

namespace moe {
int route_permute_impl(moe_ctx* ctx, const void* x, int x_dtype, const float* router_w, const float* bias,
                       const float* logits_in, int T, int H, int E, int k, float* logits_out, int32_t* topk_ids,
                       float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                       int32_t* active, void* ws, size_t ws_bytes, int32_t* ids_host, int32_t* ids_flag, int32_t seq,
                       void* stream) {
  if (!ctx) return set_error(MOE_ERR_INVALID_ARG, "moe_route_permute: ctx is NULL");
  int rc = validate_route_args("moe_route_permute", x, x_dtype, router_w, logits_in, T, H, E, k, logits_out,
                          topk_ids, topk_w);
  if (rc) return rc;
  if (!expert_offsets || !active || (T > 0 && (!sorted_pairs || !pair_pos)))
    return set_error(MOE_ERR_INVALID_ARG, "moe_route_permute: NULL grouping output");
  if ((rc = ensure_device(ctx))) return rc;
  if (!ids_host != !ids_flag) return set_error(MOE_ERR_INVALID_ARG, "moe_route_permute: host ids need their flag");
  hipStream_t s = (hipStream_t)stream;
  // Large batches, and more tokens than the fused kernel's wavefronts take
  // two at a time (it selects token by token in each wavefront; the
  // separate top-k kernel spreads the tokens over many workgroups): separate
  // kernels.  The host copy of the ids needs the fused kernel.
  if ((long long)T * k > kFusedMaxPairs || (T > kFusedMaxTokens && !ids_host)) {
    if (ids_host || ids_flag) return set_error(MOE_ERR_INVALID_ARG, "moe_route_permute: a host copy of the ids needs T*k <= %d",
                                   kFusedMaxPairs);
    rc = launch_route(ctx, x, x_dtype, router_w, bias, logits_in, T, H, E, k, logits_out, topk_ids, topk_w, s);
    if (rc) return rc;
    if (ws && !aligned(ws, 4)) return set_error(MOE_ERR_ALIGNMENT, "moe_route_permute: ws must be 4-byte aligned");
    return launch_permute(ctx, topk_ids, T * k, E, expert_offsets, sorted_pairs, pair_pos, active, ws, ws_bytes, s);
  }
  const float* src = logits_in;
  const float* tk_bias = bias;
  if (!logits_in) {
    {
      KernelTimer timer(ctx, "router_logits", s);
      launch_router_logits_kernel(x, x_dtype, router_w, bias, T, H, E, logits_out, s);
    }
    if ((rc = check_launch("router_logits_kernel"))) return rc;
    src = logits_out;
    tk_bias = nullptr;
  }
  KernelTimer timer(ctx, "topk_permute", s);
  launch(topk_permute_kernel, 1, kTopkPermuteThreads, 0, s, src, tk_bias, T, E, k, logits_in ? logits_out : nullptr, topk_ids,
                                        topk_w, expert_offsets, sorted_pairs, pair_pos, active, ctx->d_err, ids_host, ids_flag, seq);
  return check_launch("topk_permute_kernel");
}
}  // namespace moe
