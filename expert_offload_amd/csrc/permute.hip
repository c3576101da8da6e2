// Stable grouping of (token, expert) pairs by expert: LDS histogram,
// exclusive scan, then a stable scatter whose in-round ranks come from
// wavefront ballots (a "multisplit" over the expert-id bits).
#include <climits>

#include "device_common.h"

namespace moe {

constexpr int kPermThreads = 512;
constexpr int kPermWaves = kPermThreads / kWave;

// Exclusive scan of n <= kMaxE ints held in LDS `a` into LDS `out`, by one
// 512-thread block.  Returns the total to every thread.
__device__ int block_exclusive_scan(const int* a, int* out, int n, int* s_wave) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  constexpr int per = kMaxE / kPermThreads;  // 2 elements per thread
  int v[per];
  int local = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int idx = tid * per + i;
    v[i] = idx < n ? a[idx] : 0;
    local += v[i];
  }
  // inclusive wave scan of `local`
  int inc = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  if (lane == kWave - 1) s_wave[wave] = inc;
  __syncthreads();
  int wave_base = 0, total = 0;
  for (int w = 0; w < kPermWaves; ++w) {
    if (w < wave) wave_base += s_wave[w];
    total += s_wave[w];
  }
  int run = wave_base + inc - local;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int idx = tid * per + i;
    if (idx < n) out[idx] = run;
    run += v[i];
  }
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids, int P,
                                                               int E, int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_pairs,
                                                               int32_t* __restrict__ pair_pos,
                                                               int32_t* __restrict__ active,
                                                               int* __restrict__ err) {
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_cur[kMaxE];
  __shared__ int s_wcnt[kPermWaves][kMaxE];
  __shared__ int s_wave[kPermWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;

  for (int i = tid; i < kMaxE; i += kPermThreads) s_cnt[i] = 0;
  for (int i = tid; i < kPermWaves * kMaxE; i += kPermThreads) (&s_wcnt[0][0])[i] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kPermThreads) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) {
      atomicAdd(&s_cnt[e], 1);
    } else {
      atomicCAS(err, 0, INT_MIN);  // invalid expert id: the pair is left out
      pair_pos[p] = -1;
    }
  }
  __syncthreads();

  // offsets = exclusive scan of counts
  const int n_valid = block_exclusive_scan(s_cnt, s_cur, E, s_wave);
  for (int e = tid; e < E; e += kPermThreads) offsets[e] = s_cur[e];
  if (tid == 0) offsets[E] = n_valid;
  for (int i = n_valid + tid; i < P; i += kPermThreads) sorted_pairs[i] = -1;
  // active experts: exclusive scan of (count > 0) flags; s_wcnt[0] is free scratch here
  for (int e = tid; e < E; e += kPermThreads) s_wcnt[0][e] = s_cnt[e] > 0;
  __syncthreads();
  const int n_active = block_exclusive_scan(&s_wcnt[0][0], &s_wcnt[1][0], E, s_wave);
  for (int e = tid; e < E; e += kPermThreads)
    if (s_cnt[e] > 0) active[1 + s_wcnt[1][e]] = e;
  if (tid == 0) active[0] = n_active;
  __syncthreads();
  for (int i = tid; i < 2 * kMaxE; i += kPermThreads) (&s_wcnt[0][0])[i] = 0;
  int nbits = 1;
  while ((1 << nbits) <= E) ++nbits;  // ids and the sentinel E fit in nbits
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int r0 = 0; r0 < P; r0 += kPermThreads) {
    const int p = r0 + tid;
    const int id = p < P ? ids[p] : E;
    const bool valid = (unsigned)id < (unsigned)E;
    const int e = valid ? id : E;
    uint64_t match = __ballot(1);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool b = (e >> bit) & 1;
      const uint64_t m = __ballot(b);
      match &= b ? m : ~m;
    }
    const int rank = __popcll(match & lt_mask);
    if (valid && rank == 0) s_wcnt[wave][e] = __popcll(match);
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += s_wcnt[w][e];
      const int pos = s_cur[e] + pre + rank;
      sorted_pairs[pos] = p;
      pair_pos[p] = pos;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&s_cur[e], s_wcnt[wave][e]);
      s_wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
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
  permute_kernel<<<1, kPermThreads, 0, (hipStream_t)stream>>>(topk_ids, T * k, E, expert_offsets,
                                                              sorted_pairs, pair_pos, active, ctx->d_err);
  return check_launch("permute_kernel");
}
