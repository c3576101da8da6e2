// Control data of the decode expert-FFN kernels, staged in LDS: either
// read from moe_permute's results (stage_ctl) or computed in the kernel from
// the router logits (route_select, route_item, route_write).
#pragma once

#include "device_common.h"
#include "ffn.h"
#include "route_common.h"

namespace moe {

// --------------------------------------------------- control-data staging
// The grouping written by the routing launch (active list, offsets, the
// grouped pair list) and the slot table are read by every wavefront.  The
// workgroup copies them into LDS with independent loads (one memory round
// trip) instead of chasing them one dependent load at a time.
constexpr int kCtlMaxPairs = 1024;

struct CtlLds {
  int active[kMaxE + 1];
  int offsets[kMaxE + 1];
  int slots[kMaxE];
  int pairs[kCtlMaxPairs];
  float w[kCtlMaxPairs];
};

// The decode kernels run only when T*k <= kCtlMaxPairs.
template <int NT>
__device__ __forceinline__ void stage_ctl(const FfnParams& p, CtlLds& s, bool want_w) {
  const int E = p.E, P = p.T * p.k;
  for (int i = threadIdx.x; i <= E; i += NT) {
    s.active[i] = p.active[i];
    s.offsets[i] = p.offsets[i];
    if (i < E) s.slots[i] = p.slot_table[i];
  }
  for (int i = threadIdx.x; i < P; i += NT) {
    s.pairs[i] = p.sorted_pairs[i];
    if (want_w) s.w[i] = p.topk_w[i];
  }
  __syncthreads();
}

// Routing inside the gate/up kernel (T*k <= 64).  Every workgroup selects
// the top k of each token from the router logits (wavefront w takes tokens
// w, w + NT/64, ...), keeping ids, weights and each token's selection as
// bitmasks in LDS.  A wavefront then derives its work item from the masks
// alone (route_item), so no grouping pass stands between the selection and
// the weight loads; workgroup 0 groups the pairs and writes the routing
// results after its FFN work (route_write), so no barrier of the
// workgroup waits for those stores.
struct RouteLds {
  uint64_t taken[kRouteInFfnMaxPairs][kMaxE / kWave];  // per token (T <= T*k <= 64)
  int ids[kRouteInFfnMaxPairs];
  int pos[kRouteInFfnMaxPairs];
  float val[kRouteInFfnMaxPairs];  // the selected logits, (token, rank) order
};

// Threshold selection.  tau, the smallest of G >= k group maxima (groups of
// 64 / G lanes), is at most the k-th largest logit: the G maxima are G
// different logits, all >= tau.  So every member of the top k is >= tau,
// and a logit below tau outranks no logit >= tau.  The candidates (logits
// >= tau, usually about twice k) are compacted into LDS and ranked among
// themselves: the rank of a candidate is the number of candidates whose
// (logit, id) comes first (larger logit, or equal logit and smaller id), and
// a rank below k is its place in the output.  This replaces k rounds of
// wave-wide arg-max with a few DPP steps and one pass of broadcast reads.
template <int NS>
struct RankLds {
  uint64_t key[4][kWave * NS];  // per wavefront: candidate keys
};

// 64-bit key whose unsigned order puts (larger logit, then smaller id)
// first.  -0 is made +0 so that the two tie, as they do as floats.
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
  if (v == 0.0f) v = 0.0f;
  uint32_t b = __float_as_uint(v);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ float rank_key_value(uint64_t key) {
  const uint32_t b = (uint32_t)(key >> 32);
  return __uint_as_float((b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b);
}
__device__ __forceinline__ int rank_key_id(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wavefront, one token: v[i] = logit of id lane + 64 i (NaN already
// -inf), ok[i] false past E.  Writes ids[0..k) and val[0..k) (the chosen
// ids and logits by rank) and the selection bitmasks taken[0..NS), in LDS;
// cand is the wavefront's scratch of 64 * NS keys.
template <int NS>
__device__ __forceinline__ void wave_select_thresh(const float (&v)[NS], const bool (&ok)[NS], int k, int* ids,
                                                   float* val, uint64_t* taken, uint64_t* cand) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NS; ++i)
    if (ok[i]) m = fmaxf(m, v[i]);
  // group maxima over 8, 4, 2 or 1 lanes: 8, 16, 32 or 64 groups >= k
  if (k <= 32) m = fmaxf(m, dpp_f32<kDppXor1>(m));
  if (k <= 16) m = fmaxf(m, dpp_f32<kDppXor2>(m));
  if (k <= 8) m = fmaxf(m, dpp_f32<kDppHalfMirror>(m));
  float tau = fminf(m, dpp_f32<kDppXor1>(m));
  tau = fminf(tau, dpp_f32<kDppXor2>(tau));
  tau = fminf(tau, dpp_f32<kDppHalfMirror>(tau));
  tau = fminf(tau, dpp_f32<kDppMirror>(tau));
  {
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tau), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tau), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tau), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tau), 48));
    tau = fminf(fminf(r0, r1), fminf(r2, r3));
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int n = 0;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const bool c = ok[i] && v[i] >= tau;
    const uint64_t bm = __ballot(c);
    if (c) cand[n + __builtin_popcountll(bm & below)] = rank_key(v[i], lane + kWave * i);
    n += __builtin_popcountll(bm);
  }
  if (lane < NS) taken[lane] = 0;
  wave_lds_sync();
  for (int c0 = 0; c0 < n; c0 += kWave) {
    const int ci = c0 + lane;
    const uint64_t mine = ci < n ? cand[ci] : ~0ull;
    int cnt = 0;
#pragma unroll 4
    for (int j = 0; j < n; ++j) cnt += cand[j] > mine ? 1 : 0;
    if (ci < n && cnt < k) {
      const int e = rank_key_id(mine);
      ids[cnt] = e;
      val[cnt] = rank_key_value(mine);
      atomicOr(reinterpret_cast<unsigned long long*>(&taken[e / kWave]), 1ull << (e % kWave));
    }
  }
  wave_lds_sync();
}

template <int NT, int NS>
__device__ __forceinline__ void route_select(const FfnParams& p, const RouteArgs& ra, CtlLds& s, RouteLds& r,
                                             RankLds<NS>& q) {
  const int E = p.E, T = p.T, k = p.k;
  float* lo = blockIdx.x == 0 ? ra.logits_out : nullptr;
  // the slot table goes to registers first and to LDS after the selection,
  // so its loads and the logits' loads are in flight together
  constexpr int kPer = kMaxE / NT;
  int sl[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = threadIdx.x + NT * u;
    sl[u] = i < E ? p.slot_table[i] : 0;
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  for (int t = wave; t < T; t += NT / kWave) {
    const float* src = ra.logits + (size_t)t * E;
    float v[NS];
    bool ok[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int e = lane + kWave * i;
      ok[i] = e < E;
      v[i] = ok[i] ? src[e] : -INFINITY;
    }
    if (ra.bias) {
#pragma unroll
      for (int i = 0; i < NS; ++i)
        if (ok[i]) v[i] += ra.bias[lane + kWave * i];
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (ok[i] && lo) lo[(size_t)t * E + lane + kWave * i] = v[i];
      if (v[i] != v[i]) v[i] = -INFINITY;
    }
    wave_select_thresh<NS>(v, ok, k, r.ids + t * k, r.val + t * k, r.taken[t], q.key[wave]);
    // renormalised softmax over the chosen logits, lane j holding rank j:
    // the arithmetic of wave_topk_select
    const float my_val = lane < k ? r.val[t * k + lane] : -INFINITY;
    const float m0 = r.val[t * k];
    const float ex = lane < k ? expf(my_val - m0) : 0.0f;
    const float sum = wave_sum_dpp(ex);
    if (lane < k) s.w[t * k + lane] = ex / sum;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = threadIdx.x + NT * u;
    if (i < E) s.slots[i] = sl[u];
  }
  __syncthreads();
}

// Number of experts chosen by any token (uniform over the wavefront).
__device__ __forceinline__ int route_active(const RouteLds& r, int T, int E) {
  int n = 0;
  for (int i = 0; i < (E + kWave - 1) / kWave; ++i) {
    uint64_t u = 0;
    for (int t = 0; t < T; ++t) u |= r.taken[t][i];
    n += __builtin_popcountll(u);
  }
  return n;
}

// The a-th chosen expert in id order, its first place in the grouped order
// (set bits below it over all tokens) and its pairs as a bitmask over pair
// indices: set bits ascending are the stable order.  Wavefront-uniform.
struct ItemCtl {
  int e, pbeg, n_e;
  uint64_t pairs;
};
__device__ __forceinline__ ItemCtl route_item(const RouteLds& r, int T, int k, int E, int a) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int e = -1, before = 0;
  for (int i = 0; i < (E + kWave - 1) / kWave && e < 0; ++i) {
    uint64_t u = 0;
    for (int t = 0; t < T; ++t) u |= r.taken[t][i];
    const int c = __builtin_popcountll(u);
    if (a - before < c) {
      const uint64_t hit = __ballot(((u >> lane) & 1) && __builtin_popcountll(u & lt) == a - before);
      e = kWave * i + (int)__builtin_ctzll(hit);
    }
    before += c;
  }
  const int wi = e / kWave, bit = e % kWave;
  const uint64_t below = (bit == 0) ? 0ull : (~0ull >> (kWave - bit));
  int pbeg = 0;
  for (int t = 0; t < T; ++t) {
    for (int i = 0; i < wi; ++i) pbeg += __builtin_popcountll(r.taken[t][i]);
    pbeg += __builtin_popcountll(r.taken[t][wi] & below);
  }
  const uint64_t pm = __ballot(lane < T * k && r.ids[lane] == e);
  return {e, pbeg, (int)__builtin_popcountll(pm), pm};
}

template <int NT>
__device__ __forceinline__ void route_write(const FfnParams& p, const RouteArgs& ra, CtlLds& s, RouteLds& r) {
  if (threadIdx.x < kWave) wave_group_masks(r.taken, r.ids, p.T, p.k, p.E, s.pairs, r.pos, s.offsets, s.active);
  __syncthreads();
  const int P = p.T * p.k;
  for (int i = threadIdx.x; i < P; i += NT) {
    ra.ids[i] = r.ids[i];
    ra.w[i] = s.w[i];
    ra.sorted_pairs[i] = s.pairs[i];
    ra.pair_pos[i] = r.pos[i];
  }
  for (int i = threadIdx.x; i <= p.E; i += NT) ra.offsets[i] = s.offsets[i];
  for (int i = threadIdx.x; i <= s.active[0]; i += NT) ra.active[i] = s.active[i];
}

}  // namespace moe
