// Weighted combine of the per-pair expert outputs back to token order, and
// the block dequantisation entry point used by the exact-parity checks.
#include "device_common.h"

namespace moe {

// out[t][h] = sum over j ascending of w[t][j] * y[t*k + j][h].  VEC (H % 4
// == 0, y and out 16-byte aligned): each thread takes four consecutive h of
// one token with 16-byte loads; otherwise one h per thread.
template <bool VEC>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ w, int k, int H,
                                                      float* __restrict__ out) {
  const int t = blockIdx.y;
  const float* yt = y + (size_t)t * k * H;
  const float* wt = w + (size_t)t * k;
  if constexpr (VEC) {
    const int h = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (h >= H) return;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto add = [&](float wj, const float4& v) {
      acc.x = fmaf(wj, v.x, acc.x);
      acc.y = fmaf(wj, v.y, acc.y);
      acc.z = fmaf(wj, v.z, acc.z);
      acc.w = fmaf(wj, v.w, acc.w);
    };
    // the first (up to) eight pairs' rows are all requested before the
    // first product, so their latencies overlap; the sum keeps j ascending
    constexpr int kAhead = 8;
    float4 v[kAhead];
#pragma unroll
    for (int j = 0; j < kAhead; ++j)
      if (j < k) v[j] = *reinterpret_cast<const float4*>(yt + (size_t)j * H + h);
#pragma unroll
    for (int j = 0; j < kAhead; ++j)
      if (j < k) add(wt[j], v[j]);
    for (int j = kAhead; j < k; ++j) add(wt[j], *reinterpret_cast<const float4*>(yt + (size_t)j * H + h));
    *reinterpret_cast<float4*>(out + (size_t)t * H + h) = acc;
  } else {
    const int h = blockIdx.x * 256 + threadIdx.x;
    if (h >= H) return;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) acc = fmaf(wt[j], yt[(size_t)j * H + h], acc);
    out[(size_t)t * H + h] = acc;
  }
}

// One thread per block of 32 weights: exact d*q (or d*(q-8)) in fp32.
template <int QT, bool BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ packed, int rows,
                                                      int cols, void* __restrict__ out) {
  const int nblk = cols / kQK;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)rows * nblk) return;
  const int r = (int)(idx / nblk), b = (int)(idx % nblk);
  const uint8_t* row = packed + (size_t)r * row_bytes(QT, cols);
  float q[32];
  block_codes<QT>(row, b, q);
  const float d = block_scale<QT>(row, b);
  const float m = block_min<QT>(row, b);
  // d * q is exact in fp32 (11-bit scale, at most 8-bit code); with an
  // offset, d * u + m rounds once, as the format's definition does
  float wv[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) wv[i] = qtype_has_min(QT) ? fmaf(d, q[i], m) : d * q[i];
  if constexpr (BF16) {
    uint16_t* o = (uint16_t*)out + (size_t)r * cols + b * kQK;
#pragma unroll
    for (int i = 0; i < 32; ++i) o[i] = f32_to_bf16_rne(wv[i]);
  } else {
    float* o = (float*)out + (size_t)r * cols + b * kQK;
#pragma unroll
    for (int i = 0; i < 32; ++i) o[i] = wv[i];
  }
}

int launch_combine(moe_ctx* ctx, const float* y, const float* w, int T, int k, int H, float* out, hipStream_t s) {
  const bool vec = (H & 3) == 0 && aligned(y, 16) && aligned(out, 16);
  const int per = vec ? 4 * 256 : 256;  // h per workgroup
  dim3 grid((H + per - 1) / per, T);
  KernelTimer timer(ctx, "combine", s);
  if (vec) launch(combine_kernel<true>, grid, 256, 0, s, y, w, k, H, out);
  else launch(combine_kernel<false>, grid, 256, 0, s, y, w, k, H, out);
  return check_launch("combine_kernel");
}

}  // namespace moe

using namespace moe;

extern "C" int moe_combine(moe_ctx* ctx, const float* y_pairs, const float* topk_w, int T, int k,
                           int H, float* out, void* stream) {
  clear_error();
  if (!ctx) return set_error(MOE_ERR_INVALID_ARG, "moe_combine: ctx is NULL");
  if (T < 0 || k < 1 || H < 1)
    return set_error(MOE_ERR_INVALID_ARG, "moe_combine: need T >= 0, k >= 1, H >= 1 (T=%d k=%d H=%d)", T, k, H);
  if (T == 0) return MOE_OK;
  if (T > 65535) return set_error(MOE_ERR_INVALID_ARG, "moe_combine: T=%d above 65535", T);
  if (!y_pairs || !topk_w || !out) return set_error(MOE_ERR_INVALID_ARG, "moe_combine: NULL buffer");
  int rc = ensure_device(ctx);
  if (rc) return rc;
  return launch_combine(ctx, y_pairs, topk_w, T, k, H, out, (hipStream_t)stream);
}

extern "C" int moe_dequantize(moe_ctx* ctx, int qtype, const void* packed, int rows, int cols,
                              int out_dtype, void* out, void* stream) {
  clear_error();
  if (!ctx) return set_error(MOE_ERR_INVALID_ARG, "moe_dequantize: ctx is NULL");
  if (!qtype_supported(qtype))
    return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "moe_dequantize: block type %d is not supported", qtype);
  if (rows < 0 || cols <= 0 || cols % kGroupWeights)
    return set_error(MOE_ERR_INVALID_ARG, "moe_dequantize: rows=%d cols=%d (cols a multiple of %d)", rows,
                     cols, kGroupWeights);
  if (out_dtype != MOE_DTYPE_F32 && out_dtype != MOE_DTYPE_BF16)
    return set_error(MOE_ERR_INVALID_ARG, "moe_dequantize: out_dtype %d unknown", out_dtype);
  if (rows == 0) return MOE_OK;
  if (!packed || !out) return set_error(MOE_ERR_INVALID_ARG, "moe_dequantize: NULL buffer");
  if (!aligned(packed, 16)) return set_error(MOE_ERR_ALIGNMENT, "moe_dequantize: packed must be 16-byte aligned");
  int rc = ensure_device(ctx);
  if (rc) return rc;
  const long long n = (long long)rows * (cols / kQK);
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipStream_t s = (hipStream_t)stream;
  KernelTimer timer(ctx, "dequant", s);
#define MOE_DQ(Q)                                                                                           \
  case Q:                                                                                                   \
    if (out_dtype == MOE_DTYPE_F32) launch(dequant_kernel<Q, false>, grid, 256, 0, s, (const uint8_t*)packed, rows, cols, out); \
    else launch(dequant_kernel<Q, true>, grid, 256, 0, s, (const uint8_t*)packed, rows, cols, out);         \
    break;
  switch (qtype) {
    MOE_DQ(MOE_QTYPE_Q8_0)
    MOE_DQ(MOE_QTYPE_Q4_0)
    MOE_DQ(MOE_QTYPE_Q4_1)
    MOE_DQ(MOE_QTYPE_Q5_0)
    MOE_DQ(MOE_QTYPE_Q5_1)
    MOE_DQ(MOE_QTYPE_Q4_K)
    MOE_DQ(MOE_QTYPE_Q5_K)
    default: break;
  }
#undef MOE_DQ
  return check_launch("dequant_kernel");
}
