#pragma once
// Decode expert FFN on the fp32 matrix cores, for the experts that many
// tokens of a batch chose (at least kMfmaMinPairs pairs).  The GEMV kernels
// convert each weight once per token; an expert with a dozen tokens is a
// small matrix product, where v_mfma_f32_16x16x4_f32 converts each weight
// once per 16 tokens and multiplies it in the matrix cores.  The weights are
// dequantised exactly to fp32 (d times an integer code), the activations
// stay fp32, so the products are those of the GEMV kernels up to the order
// of the fp32 sums.  The GEMV kernels skip these experts (FfnParams
// mfma_min), and the down GEMV kernel's combine reads their y rows from
// memory.
//
// Tiles: a workgroup computes 16 pairs (rows) of one expert against 32
// output columns, its four wavefronts each a quarter of the K range (the
// partial sums meet in LDS): gate/up takes 16 gate and the 16 up columns of
// the same intermediate indices (SwiGLU in the accumulators), down 32
// columns of H.
// Operand layout of the instruction (lane l, 16 x 4 A, 4 x 16 B, 16 x 16 D):
// A[l % 16][l / 16], B[l / 16][l % 16], D[4 (l / 16) + r][l % 16] in r.
// The K index that lane group g = l / 16 supplies to instruction (s, q) of
// a 32-weight block is 16 s + 4 g + q, the same for A and B, so each lane
// reads four consecutive activations and four consecutive codes.
#include "decode_ctl.h"

namespace moe {

typedef float mf32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaMinPairs = 8;  // pairs of one expert from which it takes the matrix cores
// Batches from which the matrix-core kernels are launched at all: below it
// an expert with 8 pairs is rare unless the router is very skewed, and two
// launches that find no such expert cost more than they save.
constexpr int kMfmaMinBatch = 32;
constexpr int kMfmaRows = 16;     // pairs per tile

// The matrix-core kernels exist for these block types.
constexpr bool mfma_decode_type(int qt) { return qt == MOE_QTYPE_Q8_0 || qt == MOE_QTYPE_Q4_0; }

// Tiles of 16 pairs of the experts with at least kMfmaMinPairs pairs, in
// active order: tiles[a] per active expert, base[a] their exclusive scan.
struct MfmaCtl {
  int tiles[kMaxE];
  int base[kMaxE];
  int scan_wave[16];
};

template <int NT>
__device__ __forceinline__ int stage_mfma_tiles(const FfnParams& p, const CtlLds& c, MfmaCtl& m, int n_active) {
  for (int a = threadIdx.x; a < n_active; a += NT) {
    const int e = c.active[1 + a];
    const int n = c.offsets[e + 1] - c.offsets[e];
    const bool on = !(p.mask && !p.mask[e]) && n >= kMfmaMinPairs;
    m.tiles[a] = on ? (n + kMfmaRows - 1) / kMfmaRows : 0;
  }
  __syncthreads();
  return block_exclusive_scan<NT>(m.tiles, m.base, n_active, m.scan_wave);
}

// Tile t (wavefront-uniform) -> active expert a (the last with base <= t
// and tiles > 0) and the tile's first pair within the expert.
__device__ __forceinline__ void mfma_tile(const MfmaCtl& m, int n_active, int t, int& a, int& first) {
  int lo = 0, hi = n_active - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (m.base[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  a = lo;
  first = (t - m.base[a]) * kMfmaRows;
}

// Raw codes and scale of the lane's weights in block b of a row: K indices
// 4g..4g+3 (set 0) and 16+4g..16+4g+3 (set 1).
template <int QT>
struct BRaw {
  uint32_t w0, w1;  // Q4_0: w0 holds both sets (low and high nibbles)
  uint32_t d;       // fp16 bits
  __device__ __forceinline__ void load(const uint8_t* row, int b, int g) {
    const uint8_t* grp = row + (size_t)(b >> 3) * group_bytes(QT);
    const uint8_t* q = grp + (b & 7) * quant_bytes_per_block(QT);
    w0 = *reinterpret_cast<const uint32_t*>(q + 4 * g);
    if constexpr (QT == MOE_QTYPE_Q8_0) w1 = *reinterpret_cast<const uint32_t*>(q + 16 + 4 * g);
    d = *reinterpret_cast<const uint16_t*>(grp + group_d_off(QT) + 2 * (b & 7));
  }
  // weight of set s, element q: d * u - off * d for the stored code u (Q8_0:
  // q + 128, Q4_0: the nibble), one fused multiply-add of exact operands whose
  // exact result d * (u - off) is an fp32 number, so it is exact.
  __device__ __forceinline__ void dequant(float (&v)[2][4]) const {
    const float dd = __half2float(__ushort_as_half((unsigned short)d));
    const float off = -qtype_code_off(QT) * dd;
    uint32_t c0, c1;
    if constexpr (QT == MOE_QTYPE_Q8_0) {
      c0 = w0 ^ 0x80808080u;
      c1 = w1 ^ 0x80808080u;
    } else {
      c0 = w0 & 0x0F0F0F0Fu;
      c1 = (w0 >> 4) & 0x0F0F0F0Fu;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[0][q] = fmaf(dd, (float)((c0 >> (8 * q)) & 0xFFu), off);
      v[1][q] = fmaf(dd, (float)((c1 >> (8 * q)) & 0xFFu), off);
    }
  }
};

// acc[c] += rows' activations (A, 16 x K from `arow`) times the weight rows
// brow[c] (16 columns each) over blocks b_beg .. b_end - 1.  The loads run
// kDepth blocks ahead of the matrix instructions, in a ring of registers
// indexed at compile time; every load is issued on every path (no branch
// around a load), so the wait before each block counts only the loads
// issued after it and the ring stays in flight (a ring whose loads sat
// under branches waited for all of them at the loop head: 75 -> 73 us for
// gate/up and 42 -> 39 us for down at 64 tokens of 512 experts).
constexpr int kDepth = 4;
template <int QT, int NB>
__device__ __forceinline__ void mfma_rows(const float* arow, const uint8_t* const (&brow)[NB], int b_beg, int b_end,
                                          int g, mf32x4 (&acc)[NB]) {
  if (b_beg >= b_end) return;
  float4 a0[kDepth], a1[kDepth];
  BRaw<QT> raw[kDepth][NB];
  // every load unconditional (rows past the tile read a valid row; block
  // indices past the range clamp), so the wait before a block counts only
  // the loads issued after it
  auto load = [&](int u, int b) {
    b = min(b, b_end - 1);
    a0[u] = *reinterpret_cast<const float4*>(arow + 32 * b + 4 * g);
    a1[u] = *reinterpret_cast<const float4*>(arow + 32 * b + 16 + 4 * g);
#pragma unroll
    for (int c = 0; c < NB; ++c) raw[u][c].load(brow[c], b, g);
  };
  auto block = [&](int u) {
    const float av[2][4] = {{a0[u].x, a0[u].y, a0[u].z, a0[u].w}, {a1[u].x, a1[u].y, a1[u].z, a1[u].w}};
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      float wv[2][4];
      raw[u][c].dequant(wv);
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s][q], wv[s][q], acc[c], 0, 0, 0);
    }
  };
#pragma unroll
  for (int u = 0; u < kDepth; ++u) {
    load(u, b_beg + u);
    __builtin_amdgcn_sched_barrier(0);
  }
  int b0 = b_beg;
  // full groups whose successors exist: consume a slot, refill it
  for (; b0 + kDepth < b_end; b0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      block(u);
      load(u, b0 + kDepth + u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the last group: no more loads
#pragma unroll
  for (int u = 0; u < kDepth; ++u)
    if (b0 + u < b_end) block(u);
}

// A workgroup takes one tile item at a time; its four wavefronts split the
// K blocks in four consecutive ranges and their partial sums meet in LDS,
// added in wavefront order (so the result does not depend on timing).
constexpr int kSplitK = 4;
constexpr int kMfmaThreads = kWave * kSplitK;  // threads of a matrix-core workgroup
struct SplitLds {
  float part[kSplitK][2][4][kWave];
};
__device__ __forceinline__ void split_range(int nb, int w, int& b_beg, int& b_end) {
  const int per = (nb + kSplitK - 1) / kSplitK;
  b_beg = min(nb, w * per);
  b_end = min(nb, b_beg + per);
}
// The four partial sums of this lane, in wavefront order; valid in every
// wavefront after the call (two workgroup barriers).
__device__ __forceinline__ void split_reduce(SplitLds& sl, mf32x4 (&acc)[2], int w, int lane) {
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) sl.part[w][c][r][lane] = acc[c][r];
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = sl.part[0][c][r][lane];
#pragma unroll
      for (int u = 1; u < kSplitK; ++u) v += sl.part[u][c][r][lane];
      acc[c][r] = v;
    }
  __syncthreads();
}

// gate/up + SwiGLU: item = (tile, 16 intermediate indices), one per workgroup.
template <int QT>
__global__ __launch_bounds__(kMfmaThreads) void ffn_gateup_mfma(FfnParams p, const float* __restrict__ x) {
  __shared__ CtlLds ctl;
  __shared__ MfmaCtl mc;
  __shared__ SplitLds sl;
  stage_ctl<kMfmaThreads>(p, ctl, false);
  const int n_active = ctl.active[0];
  const int n_tiles = stage_mfma_tiles<kMfmaThreads>(p, ctl, mc, n_active);
  const int lane = threadIdx.x & (kWave - 1), g = lane / 16, j = lane % 16;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_chunks = p.I / 16;
  const int items = n_tiles * n_chunks;
  const size_t gate_off = slot_gate_off(QT, p.H, p.I), up_off = slot_up_off(QT, p.H, p.I);
  const size_t rbytes = row_bytes(QT, p.H);
  int b_beg, b_end;
  split_range(p.H / kQK, w, b_beg, b_end);
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int t = item / n_chunks, i0 = (item - t * n_chunks) * 16;
    int a, first;
    mfma_tile(mc, n_active, t, a, first);
    const int e = ctl.active[1 + a];
    const int pbeg = ctl.offsets[e] + first;
    const int rows = min(kMfmaRows, ctl.offsets[e + 1] - pbeg);
    const int slot = ctl.slots[e];
    if (slot < 0 || slot >= p.n_slots) {
      if (threadIdx.x == 0) atomicCAS(p.err, 0, e + 1);
      for (int s = threadIdx.x; s < rows * 16; s += kMfmaThreads) p.hbuf[(size_t)(pbeg + s / 16) * p.I + i0 + s % 16] = NAN;
      continue;
    }
    // this lane's A row: pair j of the tile (rows past the tile read pair 0's
    // row; their outputs are not stored)
    const int pair = ctl.pairs[pbeg + (j < rows ? j : 0)];
    const float* arow = x + (size_t)(pair / p.k) * p.H;
    const uint8_t* base = p.pool + (size_t)slot * p.slot_bytes;
    const uint8_t* brow[2] = {base + gate_off + (size_t)(i0 + j) * rbytes, base + up_off + (size_t)(i0 + j) * rbytes};
    mf32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    mfma_rows<QT, 2>(arow, brow, b_beg, b_end, g, acc);
    split_reduce(sl, acc, w, lane);
    if (w == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        if (i < rows) {
          const float gv = acc[0][r];
          p.hbuf[(size_t)(pbeg + i) * p.I + i0 + j] = gv / (1.0f + expf(-gv)) * acc[1][r];
        }
      }
    }
  }
}

// down: item = (tile, 32 output columns), one per workgroup; y rows in pair order.
template <int QT>
__global__ __launch_bounds__(kMfmaThreads) void ffn_down_mfma(FfnParams p) {
  __shared__ CtlLds ctl;
  __shared__ MfmaCtl mc;
  __shared__ SplitLds sl;
  stage_ctl<kMfmaThreads>(p, ctl, false);
  const int n_active = ctl.active[0];
  const int n_tiles = stage_mfma_tiles<kMfmaThreads>(p, ctl, mc, n_active);
  const int lane = threadIdx.x & (kWave - 1), g = lane / 16, j = lane % 16;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_chunks = p.H / 32;
  const int items = n_tiles * n_chunks;
  const size_t down_off = slot_down_off(QT, p.H, p.I);
  const size_t rbytes = row_bytes(QT, p.I);
  int b_beg, b_end;
  split_range(p.I / kQK, w, b_beg, b_end);
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int t = item / n_chunks, h0 = (item - t * n_chunks) * 32;
    int a, first;
    mfma_tile(mc, n_active, t, a, first);
    const int e = ctl.active[1 + a];
    const int pbeg = ctl.offsets[e] + first;
    const int rows = min(kMfmaRows, ctl.offsets[e + 1] - pbeg);
    const int slot = ctl.slots[e];
    if (slot < 0 || slot >= p.n_slots) {
      if (threadIdx.x == 0) atomicCAS(p.err, 0, e + 1);
      for (int s = threadIdx.x; s < rows * 32; s += kMfmaThreads) p.y[(size_t)ctl.pairs[pbeg + s / 32] * p.H + h0 + s % 32] = NAN;
      continue;
    }
    const float* arow = p.hbuf + (size_t)(pbeg + (j < rows ? j : 0)) * p.I;
    const uint8_t* base = p.pool + (size_t)slot * p.slot_bytes + down_off;
    const uint8_t* brow[2] = {base + (size_t)(h0 + j) * rbytes, base + (size_t)(h0 + 16 + j) * rbytes};
    mf32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    mfma_rows<QT, 2>(arow, brow, b_beg, b_end, g, acc);
    split_reduce(sl, acc, w, lane);
    if (w == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        if (i < rows) {
          float* yrow = p.y + (size_t)ctl.pairs[pbeg + i] * p.H + h0;
          yrow[j] = acc[0][r];
          yrow[16 + j] = acc[1][r];
        }
      }
    }
  }
}

}  // namespace moe
