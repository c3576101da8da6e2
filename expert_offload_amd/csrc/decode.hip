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
    default: return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "decode: block type %d", p.qtype);
  }
}

}  // namespace moe
