// Decode-path dispatch: shape support and the per-block-type launchers,
// each built in its own translation unit from decode_impl.h.
#include "decode_impl.h"

namespace moe {

bool decode_route_supported(int H, int I, int T, int k) {
  GemvShape a;
  return decode_gemv_supported(H, I, T, k) && (long long)T * k <= kRouteInFfnMaxPairs && gemv_shape(H, &a) &&
         a.lpr == 64;
}

bool decode_gemv_supported(int H, int I, int T, int k) {
  GemvShape a, b;
  return (long long)T * k <= kCtlMaxPairs && gemv_shape(H, &a) && gemv_shape(I, &b);
}

int launch_ffn_decode(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s, const RouteArgs* route) {
  switch (p.qtype) {
    case MOE_QTYPE_Q8_0: return launch_ffn_decode_q8_0(ctx, p, x, s, route);
    case MOE_QTYPE_Q4_0: return launch_ffn_decode_q4_0(ctx, p, x, s, route);
    case MOE_QTYPE_Q4_1: return launch_ffn_decode_q4_1(ctx, p, x, s, route);
    case MOE_QTYPE_Q5_0: return launch_ffn_decode_q5_0(ctx, p, x, s, route);
    case MOE_QTYPE_Q5_1: return launch_ffn_decode_q5_1(ctx, p, x, s, route);
    case MOE_QTYPE_Q4_K: return launch_ffn_decode_q4_k(ctx, p, x, s, route);
    case MOE_QTYPE_Q5_K: return launch_ffn_decode_q5_k(ctx, p, x, s, route);
    default: return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "decode: block type %d", p.qtype);
  }
}

// One thread per block of 32: s = max|v| / 127, code = v / s rounded half
// away from zero (IEEE fp32 divisions), clamped to [-127, 127]; s = 0 gives
// codes 0.  Codes go out as 32 bytes, element j in byte j.
__global__ __launch_bounds__(256) void quant_act_kernel(const float* __restrict__ src, long long n_blocks,
                                                        int8_t* __restrict__ q, float* __restrict__ s,
                                                        int* __restrict__ qsum) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= n_blocks) return;
  float v[32];
  const float4* in = reinterpret_cast<const float4*>(src + b * kQK);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 t = in[i];
    v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float sc = amax / 127.0f;
  uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    int c = sc == 0.0f ? 0 : (int)roundf(v[i] / sc);
    c = min(127, max(-127, c));
    sum += c;
    w[i >> 2] |= ((uint32_t)c & 0xFFu) << (8 * (i & 3));
  }
  uint4* out = reinterpret_cast<uint4*>(q + b * kQK);
  out[0] = make_uint4(w[0], w[1], w[2], w[3]);
  out[1] = make_uint4(w[4], w[5], w[6], w[7]);
  s[b] = sc;
  qsum[b] = sum;
}

int launch_quant_act(moe_ctx* ctx, const float* src, long long n_blocks, int8_t* q, float* s, int* qsum,
                     hipStream_t stream) {
  if (n_blocks <= 0) return MOE_OK;
  KernelTimer timer(ctx, "quant_act", stream);
  launch(quant_act_kernel, (unsigned)((n_blocks + 255) / 256), 256, 0, stream, src, n_blocks, q, s, qsum);
  return check_launch("quant_act_kernel");
}

}  // namespace moe
