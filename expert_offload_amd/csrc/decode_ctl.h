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
  int runs[kMaxE];      // pair runs of active expert a (stage_runs)
  int run_base[kMaxE];  // runs before active expert a
  int scan_wave[16];
};

// Pair runs.  With more than kRunMinTokens tokens a work item takes at most
// kRunPairs consecutive pairs of one expert, so an expert that many tokens
// chose (a skewed router) spreads over several items instead of one
// wavefront looping over all its tokens.  With fewer tokens run a is active
// expert a: no expert can have many pairs (a token names an expert once),
// and the scan in every workgroup's prologue would cost more than it saves
// (16 tokens of 128 experts: 4 us per kernel).
constexpr int kRunPairs = 8;
constexpr int kRunMinTokens = 16;

struct PairRun {
  int e, pbeg, n;  // expert, first grouped pair of the run, pairs in it
};

template <int NT>
__device__ __forceinline__ int stage_runs(const FfnParams& p, CtlLds& s, int n_active) {
  if (p.T <= kRunMinTokens) return n_active;
  for (int a = threadIdx.x; a < n_active; a += NT) {
    const int e = s.active[1 + a];
    const int n = s.offsets[e + 1] - s.offsets[e];
    s.runs[a] = p.mfma_min && n >= p.mfma_min ? 0 : (n + kRunPairs - 1) / kRunPairs;  // matrix-core experts: none
  }
  __syncthreads();
  return block_exclusive_scan<NT>(s.runs, s.run_base, n_active, s.scan_wave);
}

// Whether expert e runs on the matrix cores instead (FfnParams mfma_min).
__device__ __forceinline__ bool mfma_expert(const FfnParams& p, const CtlLds& s, int e) {
  return p.mfma_min && s.offsets[e + 1] - s.offsets[e] >= p.mfma_min;
}

// Run r (wavefront-uniform) -> its expert and pairs.  (Runs of zero pairs,
// for matrix-core experts, never come out: run_base only repeats there.)
__device__ __forceinline__ PairRun pair_run(const FfnParams& p, const CtlLds& s, int n_active, int r) {
  int a = r, first = 0;
  if (p.T > kRunMinTokens) {  // last active expert with run_base <= r
    int lo = 0, hi = n_active - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s.run_base[mid] <= r) lo = mid;
      else hi = mid - 1;
    }
    a = lo;
    first = (r - s.run_base[a]) * kRunPairs;
  }
  const int e = s.active[1 + a];
  const int pbeg = s.offsets[e];
  const int left = s.offsets[e + 1] - pbeg - first;
  return {e, pbeg + first, p.T > kRunMinTokens ? min(kRunPairs, left) : left};
}

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
};

// Per-wavefront scratch of the top-k (threshold selection).
struct RankLds {
  TopkScratch s[4];
};

template <int NT, int NS>
__device__ __forceinline__ void route_select(const FfnParams& p, const RouteArgs& ra, CtlLds& s, RouteLds& r,
                                             RankLds& q) {
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
  const int wave = threadIdx.x >> 6;
  for (int t = wave; t < T; t += NT / kWave)
    wave_topk_ns<NS>(ra.logits + (size_t)t * E, ra.bias, E, k, lo ? lo + (size_t)t * E : nullptr, nullptr, nullptr,
                     r.ids + t * k, s.w + t * k, r.taken[t], &q.s[wave]);
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
