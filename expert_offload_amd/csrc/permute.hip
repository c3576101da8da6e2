// moe_permute: stable grouping of (token, expert) pairs by expert.
//  - Up to kPermSplitMin pairs (or without a workspace): one workgroup (LDS
//    histogram, exclusive scan, ballot-ranked stable scatter).
//  - Larger batches: three launches over chunks of kPermChunk pairs.
//    1. count: each chunk's expert histogram, in LDS, to counts[chunk][E];
//    2. scan: per expert, the chunks' counts become running bases
//       (expert offset + pairs of that expert in earlier chunks); offsets
//       and the active list come from the totals;
//    3. scatter: each chunk places its pairs from its bases, ranking equal
//       ids with wavefront ballots in pair order, so the grouping stays
//       stable across chunks.
#include "route_common.h"

namespace moe {

constexpr int kPermThreads = 512;
constexpr int kPermChunk = 512;         // pairs per chunk (two rounds of 256 threads)
constexpr int kPermSplitThreads = 256;
constexpr int kPermSplitMin = 4096;     // P above this takes the chunked path

static int perm_chunks(long long P) { return (int)((P + kPermChunk - 1) / kPermChunk); }

__global__ __launch_bounds__(kPermSplitThreads) void permute_count_kernel(const int32_t* __restrict__ ids, int P,
                                                                          int E, int32_t* __restrict__ counts,
                                                                          int32_t* __restrict__ pair_pos,
                                                                          int* __restrict__ err) {
  __shared__ int cnt[kMaxE];
  for (int e = threadIdx.x; e < E; e += kPermSplitThreads) cnt[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kPermChunk, p1 = min(P, p0 + kPermChunk);
  for (int p = p0 + threadIdx.x; p < p1; p += kPermSplitThreads) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) {
      atomicAdd(&cnt[e], 1);
    } else {
      atomicCAS(err, 0, INT_MIN);
      pair_pos[p] = -1;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermSplitThreads) counts[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup of kMaxE threads: thread e walks the chunks' counts of
// expert e (reads coalesced across experts; independent loads, unrolled so
// many are in flight) and writes each chunk's base for that expert.
__global__ __launch_bounds__(kMaxE) void permute_scan_kernel(const int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ bases, int n_chunks, int P,
                                                             int E, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted_pairs,
                                                             int32_t* __restrict__ active) {
  __shared__ int tot[kMaxE], off[kMaxE], flag[kMaxE], fpos[kMaxE], wsum[kMaxE / kWave];
  const int e = threadIdx.x;
  // up to kScanRegs chunks: every count loaded at once and kept in
  // registers for the second pass (no re-read)
  constexpr int kScanRegs = 64;
  const bool in_regs = n_chunks <= kScanRegs;
  int v[kScanRegs];
  int run = 0;
  if (e < E) {
    if (in_regs) {
#pragma unroll
      for (int c = 0; c < kScanRegs; ++c) v[c] = c < n_chunks ? counts[(size_t)c * E + e] : 0;
#pragma unroll
      for (int c = 0; c < kScanRegs; ++c) run += v[c];
    } else {
#pragma unroll 16
      for (int c = 0; c < n_chunks; ++c) run += counts[(size_t)c * E + e];
    }
  }
  tot[e] = e < E ? run : 0;
  flag[e] = e < E && run > 0;
  __syncthreads();
  const int n_valid = block_exclusive_scan<kMaxE>(tot, off, E, wsum);
  const int n_active = block_exclusive_scan<kMaxE>(flag, fpos, E, wsum);
  if (e < E) {
    offsets[e] = off[e];
    if (tot[e] > 0) active[1 + fpos[e]] = e;
    int base = off[e];
    if (in_regs) {
#pragma unroll
      for (int c = 0; c < kScanRegs; ++c) {
        if (c < n_chunks) bases[(size_t)c * E + e] = base;
        base += v[c];
      }
    } else {
#pragma unroll 16
      for (int c = 0; c < n_chunks; ++c) {
        const int cv = counts[(size_t)c * E + e];
        bases[(size_t)c * E + e] = base;
        base += cv;
      }
    }
  }
  if (e == 0) {
    offsets[E] = n_valid;
    active[0] = n_active;
  }
  for (int i = n_valid + e; i < P; i += kMaxE) sorted_pairs[i] = -1;
}

__global__ __launch_bounds__(kPermSplitThreads) void permute_scatter_kernel(const int32_t* __restrict__ ids, int P,
                                                                            int E,
                                                                            const int32_t* __restrict__ bases,
                                                                            int32_t* __restrict__ sorted_pairs,
                                                                            int32_t* __restrict__ pair_pos) {
  constexpr int waves = kPermSplitThreads / kWave;
  __shared__ int cur[kMaxE];
  __shared__ int wcnt[waves][kMaxE];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  for (int e = tid; e < E; e += kPermSplitThreads) cur[e] = bases[(size_t)blockIdx.x * E + e];
  for (int i = tid; i < waves * E; i += kPermSplitThreads) wcnt[i / E][i % E] = 0;
  int nbits = 1;
  while ((1 << nbits) <= E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  __syncthreads();
  const int p0 = blockIdx.x * kPermChunk, p1 = min(P, p0 + kPermChunk);
  for (int r0 = p0; r0 < p1; r0 += kPermSplitThreads) {
    const int p = r0 + tid;
    const int id = p < p1 ? ids[p] : E;
    const bool valid = (unsigned)id < (unsigned)E;
    const int e = valid ? id : E;
    uint64_t match = __ballot(1);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool bb = (e >> bit) & 1;
      const uint64_t m = __ballot(bb);
      match &= bb ? m : ~m;
    }
    const int rank = __popcll(match & lt_mask);
    if (valid && rank == 0) wcnt[wave][e] = __popcll(match);
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
      const int pos = cur[e] + pre + rank;
      sorted_pairs[pos] = p;
      pair_pos[p] = pos;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&cur[e], wcnt[wave][e]);
      wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids, int P,
                                                               int E, int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_pairs,
                                                               int32_t* __restrict__ pair_pos,
                                                               int32_t* __restrict__ active,
                                                               int* __restrict__ err) {
  __shared__ PermuteLds<kPermThreads> s;
  block_permute<kPermThreads>(ids, P, E, offsets, sorted_pairs, pair_pos, active, err, s);
}

// counts and bases, chunks x E each
size_t permute_ws_bytes(long long P, int E) {
  return P > kPermSplitMin ? 2 * (size_t)perm_chunks(P) * E * sizeof(int32_t) : 0;
}

int launch_permute(moe_ctx* ctx, const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pairs,
                   int32_t* pair_pos, int32_t* active, void* ws, size_t ws_bytes, hipStream_t s) {
  const size_t need = permute_ws_bytes(P, E);
  if (need == 0 || !ws || ws_bytes < need) {
    KernelTimer timer(ctx, "permute", s);
    launch(permute_kernel, 1, kPermThreads, 0, s, ids, P, E, offsets, sorted_pairs, pair_pos, active, ctx->d_err);
    return check_launch("permute_kernel");
  }
  const int n_chunks = perm_chunks(P);
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* bases = counts + (size_t)n_chunks * E;
  {
    KernelTimer timer(ctx, "permute_count", s);
    launch(permute_count_kernel, n_chunks, kPermSplitThreads, 0, s, ids, P, E, counts, pair_pos, ctx->d_err);
  }
  int rc = check_launch("permute_count_kernel");
  if (rc) return rc;
  {
    KernelTimer timer(ctx, "permute_scan", s);
    launch(permute_scan_kernel, 1, kMaxE, 0, s, (const int32_t*)counts, bases, n_chunks, P, E, offsets,
           sorted_pairs, active);
  }
  if ((rc = check_launch("permute_scan_kernel"))) return rc;
  KernelTimer timer(ctx, "permute_scatter", s);
  launch(permute_scatter_kernel, n_chunks, kPermSplitThreads, 0, s, ids, P, E, (const int32_t*)bases,
         sorted_pairs, pair_pos);
  return check_launch("permute_scatter_kernel");
}

}  // namespace moe

using namespace moe;

extern "C" int moe_permute_workspace_size(int T, int k, int E, size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(MOE_ERR_INVALID_ARG, "moe_permute_workspace_size: bytes is NULL");
  if (T < 0 || k < 1 || E < 1 || E > kMaxE)
    return set_error(MOE_ERR_INVALID_ARG, "moe_permute_workspace_size: need T >= 0, k >= 1, 1 <= E <= %d", kMaxE);
  *bytes = permute_ws_bytes((long long)T * k, E);
  return MOE_OK;
}

extern "C" int moe_permute(moe_ctx* ctx, const int32_t* topk_ids, int T, int k, int E,
                           int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                           int32_t* active, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (!ctx) return set_error(MOE_ERR_INVALID_ARG, "moe_permute: ctx is NULL");
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E)
    return set_error(MOE_ERR_INVALID_ARG, "moe_permute: need T >= 0 and 1 <= k <= E <= %d (T=%d k=%d E=%d)",
                     kMaxE, T, k, E);
  if ((long long)T * k > (1ll << 30)) return set_error(MOE_ERR_INVALID_ARG, "moe_permute: T*k too large");
  if (!expert_offsets || !active || (T > 0 && (!topk_ids || !sorted_pairs || !pair_pos)))
    return set_error(MOE_ERR_INVALID_ARG, "moe_permute: NULL output");
  int rc = ensure_device(ctx);
  if (rc) return rc;
  if (ws && !aligned(ws, 4)) return set_error(MOE_ERR_ALIGNMENT, "moe_permute: ws must be 4-byte aligned");
  return launch_permute(ctx, topk_ids, T * k, E, expert_offsets, sorted_pairs, pair_pos, active, ws, ws_bytes,
                        (hipStream_t)stream);
}
