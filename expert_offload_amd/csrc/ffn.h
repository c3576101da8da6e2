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
};

int launch_ffn_valu(moe_ctx* ctx, const FfnParams& p, const void* x, int x_dtype, hipStream_t s);
bool decode_gemv_supported(int H, int I, int T, int k);
int launch_ffn_decode(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s);
bool prefill_mfma_supported(int H, int I);
size_t prefill_ws_bytes(int T, int k, int I, int E);
int launch_ffn_prefill(moe_ctx* ctx, const FfnParams& p, const void* x, void* ws, hipStream_t s);
int launch_combine(moe_ctx* ctx, const float* y, const float* w, int T, int k, int H, float* out, hipStream_t s);

}  // namespace moe
