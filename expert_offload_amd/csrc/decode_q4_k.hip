// Decode kernels for Q4_K expert banks.
#include "decode_impl.h"

namespace moe {

int launch_ffn_decode_q4_k(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s, const RouteArgs* route) {
  return launch_ffn_decode_t<MOE_QTYPE_Q4_K>(ctx, p, x, s, route);
}

}  // namespace moe
