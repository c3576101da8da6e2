// Decode kernels for Q5_0 expert banks.
#include "decode_impl.h"

namespace moe {

int launch_ffn_decode_q5_0(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s, const RouteArgs* route) {
  return launch_ffn_decode_t<MOE_QTYPE_Q5_0>(ctx, p, x, s, route);
}

}  // namespace moe
