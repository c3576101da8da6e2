// Device routines shared by the routing kernels: the wavefront top-k (a
// threshold selection, with k rounds of arg-max as the fallback) and the
// single-workgroup stable grouping of pairs by expert.
#pragma once

#include <climits>

#include "device_common.h"

namespace moe {

// One wavefront selects the top k of E values held NS = ceil(E / 64) per
// lane (slot i of lane l holds id l + 64 i; ok[i] false past E; NaN already
// replaced by -inf).  Each round takes the wave-wide maximum of the values
// still free (a 32-bit max reduction), then the lowest id holding that value
// (ballots over the slots): equal values go to the lower id.  Then w_j =
// exp(l_j - l_max) / sum_j' exp(l_j' - l_max), which equals the softmax
// probabilities renormalised over the kept experts.  Writes ids/w when set,
// also to ids_copy / w_copy if set, and with `taken` the selection as
// bitmasks: bit l of taken[i] set if expert l + 64 i was chosen (NS words).
// Chosen slots are cleared in ok.
template <int NS>
__device__ __forceinline__ void wave_topk_select(float (&v)[NS], bool (&ok)[NS], int E, int k,
                                                 int32_t* __restrict__ ids, float* __restrict__ w,
                                                 int32_t* ids_copy, float* w_copy, uint64_t* taken) {
  const int lane = threadIdx.x & (kWave - 1);
  float my_val = -INFINITY;
  for (int j = 0; j < k; ++j) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (ok[i]) m = fmaxf(m, v[i]);
    m = wave_max_dpp(m);
    int bi = -1;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const uint64_t mask = __ballot(ok[i] && v[i] == m);
      if (bi < 0 && mask) bi = (int)__builtin_ctzll(mask) + kWave * i;
    }
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (lane + kWave * i == bi) ok[i] = false;  // taken
    if (lane == j) my_val = m;
    if (lane == 0) {
      if (ids) ids[j] = bi;
      if (ids_copy) ids_copy[j] = bi;
    }
  }
  if (taken) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const uint64_t m = __ballot(lane + kWave * i < E && !ok[i]);
      if (lane == 0) taken[i] = m;
    }
  }
  const float m0 = __shfl(my_val, 0, kWave);
  const float ex = lane < k ? expf(my_val - m0) : 0.0f;
  const float s = wave_sum_dpp(ex);
  if (lane < k) {
    if (w) w[lane] = ex / s;
    if (w_copy) w_copy[lane] = ex / s;
  }
}

// ------------------------------------------------- threshold selection
// tau, the k-th largest of G >= k group maxima (groups of 64 / G lanes), is
// at most the k-th largest logit: the k largest maxima are k different
// logits, all >= tau.  So every member of the top k is >= tau, and a logit
// below tau outranks no logit >= tau.  The candidates (logits >= tau,
// usually about twice k) are compacted into LDS and ranked among
// themselves: the rank of a candidate is the number of candidates whose
// (logit, id) comes first (larger logit, or equal logit and smaller id),
// and a rank below k is its place in the output.  A few DPP steps and two
// passes of broadcast reads replace the k rounds of wave_topk_select, which
// remains the path when more than kTopkCand logits lie at or above tau.
constexpr int kTopkCand = 128;
struct TopkScratch {
  uint64_t cand[kTopkCand];
  float val[kMaxK];
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

// One wavefront: v[i] = logit of id lane + 64 i (NaN already -inf), ok[i]
// false past E.  Returns false (having written nothing) when more than
// kTopkCand logits are >= tau.  Otherwise writes ids[0..k) and ids_copy
// (each may be NULL), sc.val[0..k) (the chosen logits by rank) and, with
// `taken` (LDS), the selection bitmasks taken[0..NS).
template <int NS>
__device__ __forceinline__ bool wave_select_thresh(const float (&v)[NS], const bool (&ok)[NS], int k, int32_t* ids,
                                                   int32_t* ids_copy, uint64_t* taken, TopkScratch& sc) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NS; ++i)
    if (ok[i]) m = fmaxf(m, v[i]);
  // group maxima over 8, 4, 2 or 1 lanes: G = 8, 16, 32 or 64 groups >= k
  int gs = 1;
  if (k <= 32) { m = fmaxf(m, dpp_f32<kDppXor1>(m)); gs = 2; }
  if (k <= 16) { m = fmaxf(m, dpp_f32<kDppXor2>(m)); gs = 4; }
  if (k <= 8) { m = fmaxf(m, dpp_f32<kDppHalfMirror>(m)); gs = 8; }
  // tau = the k-th largest of the G group maxima (the smallest maximum is
  // also a bound, but a far lower one when a bias skews the logits: 40 to
  // 80 candidates instead of about 20 with E = 512, k = 10).  Ranks among
  // the maxima (ties to the lower group) go through LDS.
  const int G = kWave / gs;
  float* gmax = reinterpret_cast<float*>(sc.cand);
  if (lane % gs == 0) gmax[lane / gs] = m;
  wave_lds_sync();
  int rank = 0;
  const int g = lane / gs;
  for (int j = 0; j < G; ++j) {
    const float mj = gmax[j];
    rank += (mj > m || (mj == m && j < g)) ? 1 : 0;
  }
  const uint64_t at = __ballot(lane % gs == 0 && rank == k - 1);
  const float tau = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), (int)__builtin_ctzll(at)));
  wave_lds_sync();
  uint64_t bm[NS];
  int n = 0;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    bm[i] = __ballot(ok[i] && v[i] >= tau);
    n += __builtin_popcountll(bm[i]);
  }
  if (n > kTopkCand) return false;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int base = 0;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if ((bm[i] >> lane) & 1) sc.cand[base + __builtin_popcountll(bm[i] & below)] = rank_key(v[i], lane + kWave * i);
    base += __builtin_popcountll(bm[i]);
  }
  if (taken && lane < NS) taken[lane] = 0;
  wave_lds_sync();
  for (int c0 = 0; c0 < n; c0 += kWave) {
    const int ci = c0 + lane;
    const uint64_t mine = ci < n ? sc.cand[ci] : ~0ull;
    int cnt = 0;
#pragma unroll 4
    for (int j = 0; j < n; ++j) cnt += sc.cand[j] > mine ? 1 : 0;
    if (ci < n && cnt < k) {
      const int e = rank_key_id(mine);
      if (ids) ids[cnt] = e;
      if (ids_copy) ids_copy[cnt] = e;
      sc.val[cnt] = rank_key_value(mine);
      if (taken) atomicOr(reinterpret_cast<unsigned long long*>(&taken[e / kWave]), 1ull << (e % kWave));
    }
  }
  wave_lds_sync();
  return true;
}

// The top k of token t's E logits (src row, plus bias when given): the
// threshold selection when `scratch` (LDS) is given and the candidates fit,
// else wave_topk_select.  NaN logits count as -inf.  Writes the logits used
// to logits_out when it is set.  Both paths give the same ids and weights.
template <int NS>
__device__ __forceinline__ void wave_topk_ns(const float* __restrict__ src, const float* __restrict__ bias,
                                             int E, int k, float* __restrict__ logits_out,
                                             int32_t* __restrict__ ids, float* __restrict__ w,
                                             int32_t* ids_copy, float* w_copy = nullptr,
                                             uint64_t* taken = nullptr, TopkScratch* scratch = nullptr) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[NS];
  bool ok[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = lane + kWave * i;
    ok[i] = e < E;
    v[i] = ok[i] ? src[e] : -INFINITY;
  }
  if (bias) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (ok[i]) v[i] += bias[lane + kWave * i];
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (ok[i] && logits_out) logits_out[lane + kWave * i] = v[i];
    if (v[i] != v[i]) v[i] = -INFINITY;
  }
  if (scratch && wave_select_thresh<NS>(v, ok, k, ids, ids_copy, taken, *scratch)) {
    // renormalised softmax over the chosen logits, lane j holding rank j:
    // the arithmetic of wave_topk_select
    const float my_val = lane < k ? scratch->val[lane] : -INFINITY;
    const float m0 = scratch->val[0];
    const float ex = lane < k ? expf(my_val - m0) : 0.0f;
    const float s = wave_sum_dpp(ex);
    if (lane < k) {
      if (w) w[lane] = ex / s;
      if (w_copy) w_copy[lane] = ex / s;
    }
    return;
  }
  wave_topk_select<NS>(v, ok, E, k, ids, w, ids_copy, w_copy, taken);
}

__device__ __forceinline__ void wave_topk(const float* __restrict__ src, const float* __restrict__ bias,
                                          int E, int k, float* __restrict__ logits_out,
                                          int32_t* __restrict__ ids, float* __restrict__ w,
                                          int32_t* ids_copy, float* w_copy = nullptr,
                                          uint64_t* taken = nullptr, TopkScratch* sc = nullptr) {
  if (E <= 64) wave_topk_ns<1>(src, bias, E, k, logits_out, ids, w, ids_copy, w_copy, taken, sc);
  else if (E <= 128) wave_topk_ns<2>(src, bias, E, k, logits_out, ids, w, ids_copy, w_copy, taken, sc);
  else if (E <= 256) wave_topk_ns<4>(src, bias, E, k, logits_out, ids, w, ids_copy, w_copy, taken, sc);
  else if (E <= 512) wave_topk_ns<8>(src, bias, E, k, logits_out, ids, w, ids_copy, w_copy, taken, sc);
  else wave_topk_ns<16>(src, bias, E, k, logits_out, ids, w, ids_copy, w_copy, taken, sc);
}

// Stable grouping of the P = T*k <= 64 pairs of T tokens by one wavefront,
// from each token's selection bitmasks (taken[t][i], NW = ceil(E / 64)
// words, as wave_topk_ns writes them) and ids (ids[p] for pair p = t*k+j).
// Counting set bits replaces sorting: the pairs before expert v in the
// grouped order are the set bits below v over all tokens; a pair of token t
// follows its expert's pairs from tokens t' < t.  Writes s_sorted [P],
// s_pos [P] (place of each pair), s_offsets [E + 1] and s_active (count,
// then the experts with pairs, ascending) in LDS.
__device__ __forceinline__ void wave_group_masks(const uint64_t (*taken)[kMaxE / kWave], const int32_t* ids, int T,
                                                 int k, int E, int* s_sorted, int* s_pos, int* s_offsets,
                                                 int* s_active) {
  const int lane = threadIdx.x & (kWave - 1);
  const int NW = (E + kWave - 1) / kWave;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int base = 0, abase = 0;  // set bits of all tokens / of the union, in words below i
  for (int i = 0; i < NW; ++i) {
    int below = 0, word = 0;
    uint64_t uni = 0;
    for (int t = 0; t < T; ++t) {
      const uint64_t m = taken[t][i];
      below += __builtin_popcountll(m & lt);
      word += __builtin_popcountll(m);
      uni |= m;
    }
    const int v = lane + kWave * i;
    if (v < E) s_offsets[v] = base + below;
    if ((uni >> lane) & 1) s_active[1 + abase + __builtin_popcountll(uni & lt)] = v;
    base += word;
    abase += __builtin_popcountll(uni);
  }
  if (lane == 0) {
    s_offsets[E] = base;
    s_active[0] = abase;
  }
  const int P = T * k;
  if (lane < P) {
    const int e = ids[lane], t = lane / k;
    const int wi = e / kWave, bit = e % kWave;
    const uint64_t lo = (bit == 0) ? 0ull : (~0ull >> (kWave - bit));
    int place = 0;
    for (int tt = 0; tt < T; ++tt) {
      for (int i = 0; i < wi; ++i) place += __builtin_popcountll(taken[tt][i]);
      place += __builtin_popcountll(taken[tt][wi] & lo);
      place += tt < t ? (int)((taken[tt][wi] >> bit) & 1) : 0;
    }
    s_sorted[place] = lane;
    s_pos[lane] = place;
  }
}

// Exclusive scan of n <= kMaxE ints in LDS `a` into LDS `out` by a block of
// NT threads; returns the total.  Uses s_wave[NT / 64].
template <int NT>
__device__ int block_exclusive_scan(const int* a, int* out, int n, int* s_wave) {
  constexpr int per = kMaxE / NT;
  constexpr int waves = NT / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  int v[per];
  int local = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int idx = tid * per + i;
    v[i] = idx < n ? a[idx] : 0;
    local += v[i];
  }
  int inc = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  if (lane == kWave - 1) s_wave[wave] = inc;
  __syncthreads();
  int wave_base = 0, total = 0;
  for (int w = 0; w < waves; ++w) {
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

// LDS scratch of block_permute for NT threads.
template <int NT>
struct PermuteLds {
  int cnt[kMaxE];
  int cur[kMaxE];
  int wcnt[NT / kWave][kMaxE];
  int wave[NT / kWave];
};

// Stable grouping of the P pairs (ids[p] = expert of pair p) by one block of
// NT threads: LDS histogram, exclusive scan, then rounds of NT pairs whose
// ranks among equal ids come from wavefront ballots over the id bits plus
// per-wave counts.  Ids outside [0, E) are left out (err set to INT_MIN,
// pair_pos = -1, trailing sorted_pairs = -1).
template <int NT>
__device__ void block_permute(const int32_t* ids, int P, int E, int32_t* __restrict__ offsets,
                              int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos,
                              int32_t* __restrict__ active, int* __restrict__ err, PermuteLds<NT>& s) {
  constexpr int waves = NT / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  for (int i = tid; i < E; i += NT) s.cnt[i] = 0;
  for (int i = tid; i < waves * E; i += NT) s.wcnt[i / E][i % E] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += NT) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) {
      atomicAdd(&s.cnt[e], 1);
    } else {
      atomicCAS(err, 0, INT_MIN);
      pair_pos[p] = -1;
    }
  }
  __syncthreads();
  const int n_valid = block_exclusive_scan<NT>(s.cnt, s.cur, E, s.wave);
  for (int e = tid; e < E; e += NT) offsets[e] = s.cur[e];
  if (tid == 0) offsets[E] = n_valid;
  for (int i = n_valid + tid; i < P; i += NT) sorted_pairs[i] = -1;
  // active experts via a scan of (count > 0); wcnt rows 0 and 1 are scratch here
  static_assert(waves >= 2, "block_permute needs at least two wavefronts");
  int* flags = &s.wcnt[0][0];
  int* fpos = &s.wcnt[1][0];
  for (int e = tid; e < E; e += NT) flags[e] = s.cnt[e] > 0;
  __syncthreads();
  const int n_active = block_exclusive_scan<NT>(flags, fpos, E, s.wave);
  for (int e = tid; e < E; e += NT)
    if (s.cnt[e] > 0) active[1 + fpos[e]] = e;
  if (tid == 0) active[0] = n_active;
  __syncthreads();
  for (int i = tid; i < 2 * E; i += NT) s.wcnt[i / E][i % E] = 0;
  int nbits = 1;
  while ((1 << nbits) <= E) ++nbits;
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int r0 = 0; r0 < P; r0 += NT) {
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
    if (valid && rank == 0) s.wcnt[wave][e] = __popcll(match);
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += s.wcnt[w][e];
      const int pos = s.cur[e] + pre + rank;
      sorted_pairs[pos] = p;
      pair_pos[p] = pos;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&s.cur[e], s.wcnt[wave][e]);
      s.wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

// Stable grouping by the first wavefront of the block alone (no barriers),
// for P <= 1024 pairs: LDS histogram, a wave-level exclusive scan over the
// experts (each lane owns ceil(E/64) consecutive ids), then rounds of 64
// pairs ranked by ballots over the id bits and a per-expert LDS cursor.
// cnt and cur are LDS arrays of >= E ints.  Same outputs as block_permute.
__device__ void wave_permute(const int32_t* ids, int P, int E, int32_t* __restrict__ offsets,
                             int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos,
                             int32_t* __restrict__ active, int* __restrict__ err, int* cnt, int* cur) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int e = lane; e < E; e += kWave) cnt[e] = 0;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  for (int p = lane; p < P; p += kWave) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) {
      atomicAdd(&cnt[e], 1);
    } else {
      atomicCAS(err, 0, INT_MIN);
      pair_pos[p] = -1;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const int per = (E + kWave - 1) / kWave;
  const int e0 = lane * per;
  int tot = 0, nz = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      tot += cnt[e];
      nz += cnt[e] > 0;
    }
  }
  int inc_t = tot, inc_n = nz;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int a = __shfl_up(inc_t, off, kWave), b = __shfl_up(inc_n, off, kWave);
    if (lane >= off) {
      inc_t += a;
      inc_n += b;
    }
  }
  int run = inc_t - tot, arun = inc_n - nz;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int c = cnt[e];
      offsets[e] = run;
      cur[e] = run;
      if (c > 0) active[1 + arun++] = e;
      run += c;
    }
  }
  const int n_valid = __shfl(inc_t, kWave - 1, kWave);
  const int n_act = __shfl(inc_n, kWave - 1, kWave);
  if (lane == 0) {
    offsets[E] = n_valid;
    active[0] = n_act;
  }
  for (int i = n_valid + lane; i < P; i += kWave) sorted_pairs[i] = -1;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  int nbits = 1;
  while ((1 << nbits) <= E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int r0 = 0; r0 < P; r0 += kWave) {
    const int p = r0 + lane;
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
    if (valid) {
      const int pos = cur[e] + rank;
      sorted_pairs[pos] = p;
      pair_pos[p] = pos;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (valid && rank == 0) cur[e] += __popcll(match);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
}

}  // namespace moe
