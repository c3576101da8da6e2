// moe_permute: stable grouping of (token, expert) pairs by expert in one
// workgroup (LDS histogram, exclusive scan, ballot-ranked stable scatter).
#include "route_common.h"

namespace moe {

constexpr int kPermThreads = 512;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids, int P,
                                                               int E, int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_pairs,
                                                               int32_t* __restrict__ pair_pos,
                                                               int32_t* __restrict__ active,
                                                               int* __restrict__ err) {
  __shared__ PermuteLds<kPermThreads> s;
  block_permute<kPermThreads>(ids, P, E, offsets, sorted_pairs, pair_pos, active, err, s);
}

int launch_permute(moe_ctx* ctx, const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pairs,
                   int32_t* pair_pos, int32_t* active, hipStream_t s) {
  KernelTimer timer(ctx, "permute", s);
  launch(permute_kernel, 1, kPermThreads, 0, s, ids, P, E, offsets, sorted_pairs, pair_pos, active, ctx->d_err);
  return check_launch("permute_kernel");
}

}  // namespace moe

using namespace moe;

extern "C" int moe_permute_workspace_size(int T, int k, int E, size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(MOE_ERR_INVALID_ARG, "moe_permute_workspace_size: bytes is NULL");
  (void)T; (void)k; (void)E;
  *bytes = 0;
  return MOE_OK;
}

extern "C" int moe_permute(moe_ctx* ctx, const int32_t* topk_ids, int T, int k, int E,
                           int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                           int32_t* active, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  (void)ws; (void)ws_bytes;
  if (!ctx) return set_error(MOE_ERR_INVALID_ARG, "moe_permute: ctx is NULL");
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E)
    return set_error(MOE_ERR_INVALID_ARG, "moe_permute: need T >= 0 and 1 <= k <= E <= %d (T=%d k=%d E=%d)",
                     kMaxE, T, k, E);
  if ((long long)T * k > (1ll << 30)) return set_error(MOE_ERR_INVALID_ARG, "moe_permute: T*k too large");
  if (!expert_offsets || !active || (T > 0 && (!topk_ids || !sorted_pairs || !pair_pos)))
    return set_error(MOE_ERR_INVALID_ARG, "moe_permute: NULL output");
  int rc = ensure_device(ctx);
  if (rc) return rc;
  return launch_permute(ctx, topk_ids, T * k, E, expert_offsets, sorted_pairs, pair_pos, active,
                        (hipStream_t)stream);
}
