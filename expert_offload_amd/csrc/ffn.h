// Expert-FFN launch parameters shared by the kernel families.
#pragma once

#include "moe_internal.h"

namespace moe {

struct FfnParams {
  const uint8_t* pool;
  size_t slot_bytes;
  int n_slots;
  int qtype;
  int H, I, T, k, E;
  const int32_t* slot_table;
  const int32_t* offsets;
  const int32_t* sorted_pairs;
  const int32_t* active;
  const int32_t* mask;
  float* y;     // [T*k][H] fp32, pair order
  float* hbuf;  // [T*k][I] fp32, grouped (sorted) order
  int* err;
  const float* topk_w;  // [T][k] (fused combine only)
  float* out;           // [T][H] or NULL: fused combine target
  // int8 activations (MOE_MODE_DECODE_Q8A), else NULL: per 32-block codes,
  // scales and code sums of x [T][H] and of the h rows [T*k][I] (grouped)
  int8_t* xq;
  float* xs;
  int* xsum;
  int8_t* hq;
  float* hs;
  int* hsum;
  // experts with at least this many pairs run on the matrix cores (their
  // own kernels), and the GEMV kernels skip them; 0: none
  int mfma_min = 0;
};

// Routing done inside the decode gate/up kernel (small batches, T*k <= 64):
// every workgroup selects the top k of each token from `logits` (+ bias)
// and groups the pairs in LDS; workgroup 0 also writes the results.
struct RouteArgs {
  const float* logits;   // [T][E]
  const float* bias;     // [E] or NULL
  float* logits_out;     // [T][E] biased logits, or NULL
  int32_t* ids;          // [T][k]
  float* w;              // [T][k]
  int32_t* offsets;      // [E + 1]
  int32_t* sorted_pairs; // [T*k]
  int32_t* pair_pos;     // [T*k]
  int32_t* active;       // [1 + E]
};
constexpr int kRouteInFfnMaxPairs = 64;

int launch_ffn_valu(moe_ctx* ctx, const FfnParams& p, const void* x, int x_dtype, hipStream_t s);
bool decode_gemv_supported(int H, int I, int T, int k);
bool decode_route_supported(int H, int I, int T, int k);
int launch_ffn_decode_q8_0(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s, const RouteArgs* route);
int launch_ffn_decode_q4_0(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s, const RouteArgs* route);
int launch_ffn_decode_q4_1(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s, const RouteArgs* route);
int launch_ffn_decode_q5_0(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s, const RouteArgs* route);
int launch_ffn_decode_q5_1(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s, const RouteArgs* route);
int launch_ffn_decode_q4_k(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s, const RouteArgs* route);
int launch_ffn_decode_q5_k(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s, const RouteArgs* route);
int launch_ffn_decode(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s,
                      const RouteArgs* route = nullptr);
// int8 block quantisation of n_blocks blocks of 32 floats at src (rows laid
// end to end): codes q, scales s = max|v| / 127 and code sums.
int launch_quant_act(moe_ctx* ctx, const float* src, long long n_blocks, int8_t* q, float* s, int* qsum,
                     hipStream_t stream);
bool prefill_mfma_supported(int H, int I);
size_t prefill_ws_bytes(int T, int k, int I, int E);
int launch_ffn_prefill(moe_ctx* ctx, const FfnParams& p, const void* x, void* ws, hipStream_t s);
// moe_route_permute with an optional copy of the ids written straight into
// coherent pinned host memory by the routing kernel, which then stores seq
// into *ids_flag (both or neither); needs T*k <= 4096.
int route_permute_impl(moe_ctx* ctx, const void* x, int x_dtype, const float* router_w, const float* bias,
                       const float* logits_in, int T, int H, int E, int k, float* logits_out, int32_t* topk_ids,
                       float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                       int32_t* active, void* ws, size_t ws_bytes, int32_t* ids_host, int32_t* ids_flag,
                       int32_t seq, void* stream);
int validate_route_args(const char* fn, const void* x, int x_dtype, const float* router_w,
                        const float* logits_in, int T, int H, int E, int k, float* logits_out,
                        int32_t* topk_ids, float* topk_w);
int launch_router_logits(moe_ctx* ctx, const void* x, int x_dtype, const float* router_w, const float* bias, int T,
                         int H, int E, float* logits_out, hipStream_t s);
int launch_combine(moe_ctx* ctx, const float* y, const float* w, int T, int k, int H, float* out, hipStream_t s);

}  // namespace moe
