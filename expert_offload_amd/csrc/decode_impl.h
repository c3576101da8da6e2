#pragma once
// Decode-path kernels: the expert FFN as HBM-streaming dequant-GEMVs
// (gate/up + SwiGLU, then down + combine), with the routing optionally done
// inside the gate/up kernel.  The GEMV building blocks are in decode_gemv.h.
// Templates only: each block type is instantiated in its own translation
// unit (decode_<type>.hip) so the five build in parallel.
#include <climits>

#include "device_common.h"
#include "ffn.h"
#include "decode_ctl.h"
#include "decode_gemv.h"
#include "route_common.h"
#include "decode_mfma.h"

namespace moe {

// ------------------------------------------------------ gate/up + SwiGLU
// A work item is one wavefront: (active expert, RW/2 intermediate indices);
// its rows interleave gate and up: row 2m = gate(i0 + m), 2m + 1 = up(i0 + m).
// RNS = 0: control data from moe_permute's results; RNS > 0: routing in the
// kernel, with ceil(E / 64) <= RNS logits per lane in the top-k.
// AQ: int8 activations (MOE_MODE_DECODE_Q8A), from p.xq / p.xs / p.xsum.
template <int QT, int LPR, int BPL, int RPL, int RNS, bool AQ = false>
__global__ __launch_bounds__(256) void ffn_gateup_decode(FfnParams p, const float* __restrict__ x, RouteArgs ra) {
  constexpr bool ROUTE = RNS > 0;
  constexpr int RPP = kWave / LPR, RW = RPP * RPL, NI = RW / 2;
  __shared__ CtlLds ctl;
  __shared__ RouteLds rlds;
  __shared__ RankLds rank_lds;
  int n_active;
  if constexpr (ROUTE) {
    route_select<256, RNS>(p, ra, ctl, rlds, rank_lds);
    n_active = route_active(rlds, p.T, p.E);
  } else {
    stage_ctl<256>(p, ctl, false);
    n_active = stage_runs<256>(p, ctl, ctl.active[0]);  // pair runs (one per expert up to kRunPairs tokens)
  }
  const int* pairs = ctl.pairs;
  constexpr int STRIDE = RPL >= 2 ? LPR / RPL : LPR;  // lane distance gate row -> up row
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / LPR, lg = lane % LPR;
  const int rr = g * RPL + lg / (LPR / RPL);  // row this lane holds after the fold
  const bool writer = (lg % (LPR / RPL)) == 0 && (rr & 1) == 0;
  const int n_chunks = p.I / NI;
  const int items = n_active * n_chunks;
  const size_t gate_off = slot_gate_off(QT, p.H, p.I), up_off = slot_up_off(QT, p.H, p.I);
  const size_t rbytes = row_bytes(QT, p.H);
  for (int item = blockIdx.x * 4 + (threadIdx.x >> 6); item < items; item += gridDim.x * 4) {
    const int a = item / n_chunks, c = item - a * n_chunks;
    int e, pbeg, n_e;
    uint64_t pm = 0;  // routing variant: the expert's pairs as bits
    if constexpr (ROUTE) {
      const ItemCtl ic = route_item(rlds, p.T, p.k, p.E, a);
      e = ic.e;
      pbeg = ic.pbeg;
      n_e = ic.n_e;
      pm = ic.pairs;
    } else {
      const PairRun run = pair_run(p, ctl, ctl.active[0], a);
      e = run.e;
      pbeg = run.pbeg;
      n_e = run.n;
      if (mfma_expert(p, ctl, e)) continue;  // on the matrix cores
    }
    // pair s of the expert, s = 0, 1, ... in turn
    int s_next = 0;
    auto next_pair = [&]() -> int {
      if constexpr (ROUTE) {
        const int q = (int)__builtin_ctzll(pm);
        pm &= pm - 1;
        return q;
      } else {
        return pairs[pbeg + s_next++];
      }
    };
    if (p.mask && !p.mask[e]) continue;
    const int slot = ctl.slots[e];
    const int i0 = c * NI;
    if (slot < 0 || slot >= p.n_slots) {
      if (lane == 0) atomicCAS(p.err, 0, e + 1);
      for (int s = lane; s < n_e * NI; s += kWave) p.hbuf[(size_t)(pbeg + s / NI) * p.I + i0 + s % NI] = NAN;
      continue;
    }
    const uint8_t* base = p.pool + (size_t)slot * p.slot_bytes;
    const uint8_t* rows[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int rw = g * RPL + r;
      rows[r] = base + ((rw & 1) ? up_off : gate_off) + (size_t)(i0 + rw / 2) * rbytes;
    }
    auto finish = [&](int s, float (&acc)[RPL]) {
      fold_rows<LPR / 2, RPL, RPL>(acc, lane);
      const float u = __shfl_down(acc[0], STRIDE, kWave);
      if (writer) {
        const float gv = acc[0];
        p.hbuf[(size_t)(pbeg + s) * p.I + i0 + rr / 2] = gv / (1.0f + expf(-gv)) * u;
      }
    };
    RowTile<QT, LPR, BPL, RPL> tile;
    if constexpr (AQ) {
      const int nb = p.H / kQK;
      ActQ8<LPR, BPL> a;
      int tok = next_pair() / p.k;
      a.load(p.xq + (size_t)tok * p.H, p.xs + (size_t)tok * nb, p.xsum + (size_t)tok * nb, lg);
      tile.load(rows, lg);
      for (int s = 0; s < n_e; ++s) {
        if (s) {
          tok = next_pair() / p.k;
          a.load(p.xq + (size_t)tok * p.H, p.xs + (size_t)tok * nb, p.xsum + (size_t)tok * nb, lg);
        }
        float acc[RPL];
        tile.dot_q8(a, acc);
        finish(s, acc);
      }
    } else {
      // the first token's activations go out before the weights (L2 hits),
      // and the first token is peeled out of the loop so its row-by-row
      // waits cover only the weight loads issued so far
      float xv[BPL][32];
      load_act<LPR, BPL>(x + (size_t)(next_pair() / p.k) * p.H, lg, xv);
      tile.load(rows, lg);
      {
        float acc[RPL];
        tile.dot(xv, acc);
        finish(0, acc);
      }
      for (int s = 1; s < n_e; ++s) {
        load_act<LPR, BPL>(x + (size_t)(next_pair() / p.k) * p.H, lg, xv);
        float acc[RPL];
        tile.dot(xv, acc);
        finish(s, acc);
      }
    }
  }
  if constexpr (ROUTE) {
    if (blockIdx.x == 0) route_write<256>(p, ra, ctl, rlds);
  }
}

// ------------------------------------------------------ down (+ combine)
// A workgroup owns RW output rows of every active expert; its wavefronts
// take the experts in turn (expert a -> wave a mod waves), write y for their
// pairs, and after a barrier the workgroup forms out[t] = sum_j w[t][j] *
// y[t*k + j] over those rows (j ascending, as moe_combine does).  No data
// crosses workgroups, so no device-wide fences are needed.

// Wavefronts per down workgroup: 16 where one row per lane and activations
// streamed from LDS keep a wavefront within 128 registers (four per SIMD),
// else 8.
template <int QT, int LPR, int BPL, int RPL>
constexpr int down_waves() {
  constexpr bool stream = kWave / LPR > 1 && kQK * LPR * BPL <= kDownStageFloats && RPL == 1;
  return stream && !QTraits<QT>::kQh ? 16 : kDownWaves;
}

template <int QT, int LPR, int BPL, int RPL, bool AQ = false>
__global__ __launch_bounds__((down_waves<QT, LPR, BPL, RPL>() * kWave)) void ffn_down_decode(FfnParams p) {
  constexpr int RPP = kWave / LPR, RW = RPP * RPL;
  constexpr int NWV = down_waves<QT, LPR, BPL, RPL>();
  __shared__ float s_y[kDownLdsFloats];
  __shared__ float s_h[NWV][kDownStageFloats];
  __shared__ CtlLds ctl;
  stage_ctl<NWV * kWave>(p, ctl, p.out != nullptr);
  const int* pairs = ctl.pairs;
  const float* topk_w = ctl.w;
  // (with matrix-core experts, their y rows are read back from memory)
  const bool lds_y = p.T * p.k * RW <= kDownLdsFloats && !p.mfma_min;
  // With LPR < 64 the 64/LPR lane groups own the same columns of h: each h
  // row is read from memory once (issued before the weights) into the
  // wavefront's LDS row, and the groups read their blocks from there.
  // (the kernel for LPR lanes of BPL blocks serves I = 32 * LPR * BPL only)
  constexpr bool stage_h = !AQ && RPP > 1 && kQK * LPR * BPL <= kDownStageFloats;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  float* hrow = s_h[wave];
  const int g = lane / LPR, lg = lane % LPR;
  const int rr = g * RPL + lg / (LPR / RPL);
  const bool writer = (lg % (LPR / RPL)) == 0;
  const int n_tiles = p.H / RW;
  const int n_active = ctl.active[0];
  const int n_runs = stage_runs<NWV * kWave>(p, ctl, n_active);  // pair runs of at most kRunPairs pairs
  const size_t down_off = slot_down_off(QT, p.H, p.I);
  const size_t rbytes = row_bytes(QT, p.I);
  for (int tile_i = blockIdx.x; tile_i < n_tiles; tile_i += gridDim.x) {
    const int h0 = tile_i * RW;
    for (int r = wave; r < n_runs; r += NWV) {
      const PairRun run = pair_run(p, ctl, n_active, r);
      const int e = run.e;
      if (p.mask && !p.mask[e]) continue;
      if (mfma_expert(p, ctl, e)) continue;  // its y rows come from the matrix-core kernel
      const int slot = ctl.slots[e];
      const int pbeg = run.pbeg, n_e = run.n;
      if (slot < 0 || slot >= p.n_slots) {
        if (lane == 0) atomicCAS(p.err, 0, e + 1);
        for (int s = lane; s < n_e * RW; s += kWave) {
          const int pair = pairs[pbeg + s / RW];
          p.y[(size_t)pair * p.H + h0 + s % RW] = NAN;
          if (lds_y) s_y[pair * RW + s % RW] = NAN;
        }
        continue;
      }
      const uint8_t* base = p.pool + (size_t)slot * p.slot_bytes + down_off;
      const uint8_t* rows[RPL];
#pragma unroll
      for (int r = 0; r < RPL; ++r) rows[r] = base + (size_t)(h0 + g * RPL + r) * rbytes;
#define MOE_DOWN_FINISH(S)                                  \
  do {                                                      \
    const int pair_ = pairs[pbeg + (S)];                    \
    fold_rows<LPR / 2, RPL, RPL>(acc, lane);                \
    if (writer) {                                           \
      p.y[(size_t)pair_ * p.H + h0 + rr] = acc[0];          \
      if (lds_y) s_y[pair_ * RW + rr] = acc[0];             \
    }                                                       \
  } while (0)
      RowTile<QT, LPR, BPL, RPL, true> tile;
      float xv[BPL][32];
      if constexpr (stage_h) {
        HRowRegs hr;
        hr.load(p.hbuf + (size_t)pbeg * p.I, p.I, lane);
        tile.load(rows, lg);
        hr.store(hrow, p.I, lane);
        // one row per lane: activations straight from LDS, a block at a time
        auto dot_h = [&](float (&acc)[RPL]) {
          if constexpr (RPL == 1) tile.dot_lds_swz(hrow, lg, acc);
          else {
            load_act_swz<LPR, BPL>(hrow, lg, xv);
            tile.dot(xv, acc);
          }
        };
        float acc[RPL];
        dot_h(acc);
        MOE_DOWN_FINISH(0);
        for (int s = 1; s < n_e; ++s) {
          hr.load(p.hbuf + (size_t)(pbeg + s) * p.I, p.I, lane);
          hr.store(hrow, p.I, lane);
          dot_h(acc);
          MOE_DOWN_FINISH(s);
        }
      } else if constexpr (AQ) {
        const int nb = p.I / kQK;
        ActQ8<LPR, BPL> a;
        a.load(p.hq + (size_t)pbeg * p.I, p.hs + (size_t)pbeg * nb, p.hsum + (size_t)pbeg * nb, lg);
        tile.load(rows, lg);
        float acc[RPL];
        tile.dot_q8(a, acc);
        MOE_DOWN_FINISH(0);
        for (int s = 1; s < n_e; ++s) {
          a.load(p.hq + (size_t)(pbeg + s) * p.I, p.hs + (size_t)(pbeg + s) * nb, p.hsum + (size_t)(pbeg + s) * nb, lg);
          tile.dot_q8(a, acc);
          MOE_DOWN_FINISH(s);
        }
      } else {
        load_act<LPR, BPL>(p.hbuf + (size_t)pbeg * p.I, lg, xv);
        tile.load(rows, lg);
        float acc[RPL];
        tile.dot(xv, acc);
        MOE_DOWN_FINISH(0);
        for (int s = 1; s < n_e; ++s) {
          load_act<LPR, BPL>(p.hbuf + (size_t)(pbeg + s) * p.I, lg, xv);
          tile.dot(xv, acc);
          MOE_DOWN_FINISH(s);
        }
      }
#undef MOE_DOWN_FINISH
    }
    if (p.out) {
      __syncthreads();
      for (int idx = threadIdx.x; idx < p.T * RW; idx += NWV * kWave) {
        const int t = idx / RW, r = idx - t * RW;
        float acc = 0.0f;
        for (int j = 0; j < p.k; ++j) {
          const float yv = lds_y ? s_y[(t * p.k + j) * RW + r] : p.y[((size_t)t * p.k + j) * p.H + h0 + r];
          acc = fmaf(topk_w[(size_t)t * p.k + j], yv, acc);
        }
        p.out[(size_t)t * p.H + h0 + r] = acc;
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------ dispatch
struct GemvShape {
  int lpr, bpl;
};

// Lanes per row: every block of a row is owned by one of LPR lanes, each
// holding BPL blocks.  Returns false for column counts without a kernel.
inline bool gemv_shape(int cols, GemvShape* s) {
  const int nblk = cols / kQK;
  for (int lpr = 64; lpr >= 8; lpr >>= 1) {
    if (nblk % lpr == 0 && nblk / lpr <= 3) {
      *s = {lpr, nblk / lpr};
      return true;
    }
  }
  return false;
}


// Rows per lane of the gate/up kernel without routing inside, for 8 tokens
// and more (gateup_wide_rows): twice the register budget (up to 16), so
// each activation block, its sum and the per-pair fold serve twice the
// rows.  Fewer tokens keep the narrower rows: their few experts need the
// wider spread of work items.
inline bool gateup_wide_rows(int T, bool route) { return !route && T >= 8; }
template <int QT, int LPR, int BPL>
static constexpr int gateup_batch_rpl() {
  constexpr int RPL0 = rows_per_lane<QT, BPL>();
  constexpr int RPL = RPL0 > LPR ? LPR : RPL0;
  return 2 * RPL <= LPR && 2 * RPL <= 16 ? 2 * RPL : RPL;
}

template <int QT, int LPR, int BPL, bool AQ = false>
static void launch_gateup(const FfnParams& p, const float* x, int grid, hipStream_t s, const RouteArgs* ra) {
  constexpr int RPL0 = rows_per_lane<QT, BPL>();
  constexpr int RPL = RPL0 > LPR ? LPR : RPL0;
  if (AQ || !ra) {
    constexpr int RPLB = gateup_batch_rpl<QT, LPR, BPL>();
    if (gateup_wide_rows(p.T, false))
      launch(ffn_gateup_decode<QT, LPR, BPL, RPLB, 0, AQ>, grid, 256, 0, s, p, x, RouteArgs{});
    else
      launch(ffn_gateup_decode<QT, LPR, BPL, RPL, 0, AQ>, grid, 256, 0, s, p, x, RouteArgs{});
    return;
  }
  if constexpr (LPR == 64) {  // the routing variant exists for these shapes (decode_route_supported)
    if (p.E <= 64) launch(ffn_gateup_decode<QT, LPR, BPL, RPL, 1>, grid, 256, 0, s, p, x, *ra);
    else if (p.E <= 128) launch(ffn_gateup_decode<QT, LPR, BPL, RPL, 2>, grid, 256, 0, s, p, x, *ra);
    else if (p.E <= 256) launch(ffn_gateup_decode<QT, LPR, BPL, RPL, 4>, grid, 256, 0, s, p, x, *ra);
    else if (p.E <= 512) launch(ffn_gateup_decode<QT, LPR, BPL, RPL, 8>, grid, 256, 0, s, p, x, *ra);
    else launch(ffn_gateup_decode<QT, LPR, BPL, RPL, 16>, grid, 256, 0, s, p, x, *ra);
  }
}
template <int QT, int LPR, int BPL, bool AQ = false>
static void launch_down(const FfnParams& p, int grid, hipStream_t s) {
  constexpr int rpl = down_rows_per_lane<QT, LPR, BPL>();
  launch(ffn_down_decode<QT, LPR, BPL, rpl, AQ>, grid, down_waves<QT, LPR, BPL, rpl>() * kWave, 0, s, p);
}
template <int QT, int LPR, int BPL>
static constexpr int down_rows_per_tile() {
  return (kWave / LPR) * down_rows_per_lane<QT, LPR, BPL>();
}
template <int QT, int LPR, int BPL>
static constexpr int rows_per_wave() {
  constexpr int RPL0 = rows_per_lane<QT, BPL>();
  constexpr int RPL = RPL0 > LPR ? LPR : RPL0;
  return (kWave / LPR) * RPL;
}

template <int QT>
static int down_rows_rt(GemvShape sh) {
#define MOE_RPT(L, B) \
  if (sh.lpr == L && sh.bpl == B) return down_rows_per_tile<QT, L, B>();
  MOE_RPT(64, 1) MOE_RPT(64, 2) MOE_RPT(64, 3) MOE_RPT(32, 1) MOE_RPT(32, 2) MOE_RPT(32, 3)
  MOE_RPT(16, 1) MOE_RPT(16, 2) MOE_RPT(16, 3) MOE_RPT(8, 1) MOE_RPT(8, 2) MOE_RPT(8, 3)
#undef MOE_RPT
  return 0;
}

template <int QT>
static int batch_rows_per_wave_rt(GemvShape sh) {
#define MOE_RPW(L, B) \
  if (sh.lpr == L && sh.bpl == B) return (kWave / L) * gateup_batch_rpl<QT, L, B>();
  MOE_RPW(64, 1) MOE_RPW(64, 2) MOE_RPW(64, 3) MOE_RPW(32, 1) MOE_RPW(32, 2) MOE_RPW(32, 3)
  MOE_RPW(16, 1) MOE_RPW(16, 2) MOE_RPW(16, 3) MOE_RPW(8, 1) MOE_RPW(8, 2) MOE_RPW(8, 3)
#undef MOE_RPW
  return 0;
}

template <int QT>
static int rows_per_wave_rt(GemvShape sh) {
#define MOE_RPW(L, B) \
  if (sh.lpr == L && sh.bpl == B) return rows_per_wave<QT, L, B>();
  MOE_RPW(64, 1) MOE_RPW(64, 2) MOE_RPW(64, 3) MOE_RPW(32, 1) MOE_RPW(32, 2) MOE_RPW(32, 3)
  MOE_RPW(16, 1) MOE_RPW(16, 2) MOE_RPW(16, 3) MOE_RPW(8, 1) MOE_RPW(8, 2) MOE_RPW(8, 3)
#undef MOE_RPW
  return 0;
}

template <int QT, bool AQ = false>
static void dispatch_gateup(GemvShape sh, const FfnParams& p, const float* x, int grid, hipStream_t s,
                            const RouteArgs* ra) {
#define MOE_GU(L, B) \
  if (sh.lpr == L && sh.bpl == B) return launch_gateup<QT, L, B, AQ>(p, x, grid, s, ra);
  MOE_GU(64, 1) MOE_GU(64, 2) MOE_GU(64, 3) MOE_GU(32, 1) MOE_GU(32, 2) MOE_GU(32, 3)
  MOE_GU(16, 1) MOE_GU(16, 2) MOE_GU(16, 3) MOE_GU(8, 1) MOE_GU(8, 2) MOE_GU(8, 3)
#undef MOE_GU
}
template <int QT, bool AQ = false>
static void dispatch_down(GemvShape sh, const FfnParams& p, int grid, hipStream_t s) {
#define MOE_DN(L, B) \
  if (sh.lpr == L && sh.bpl == B) return launch_down<QT, L, B, AQ>(p, grid, s);
  MOE_DN(64, 1) MOE_DN(64, 2) MOE_DN(64, 3) MOE_DN(32, 1) MOE_DN(32, 2) MOE_DN(32, 3)
  MOE_DN(16, 1) MOE_DN(16, 2) MOE_DN(16, 3) MOE_DN(8, 1) MOE_DN(8, 2) MOE_DN(8, 3)
#undef MOE_DN
}

template <int QT>
int launch_ffn_decode_t(moe_ctx* ctx, const FfnParams& p, const float* x, hipStream_t s, const RouteArgs* route) {
  GemvShape gu, dn;
  gemv_shape(p.H, &gu);
  gemv_shape(p.I, &dn);
  const int max_active = std::min(p.E, p.T * p.k);
  // the routed kernel repeats the top-k in every workgroup: no more
  // workgroups than are resident at once (three per CU), which then take
  // further items in turn
  const int cap = (route ? 3 : 16) * ctx->num_cus;
  const int rw_gu =
      gateup_wide_rows(p.T, route != nullptr) ? batch_rows_per_wave_rt<QT>(gu) : rows_per_wave_rt<QT>(gu);
  const int rt_dn = down_rows_rt<QT>(dn);
  const long long items_gu = (long long)max_active * (p.I / (rw_gu / 2));
  const int grid_gu = (int)std::max(1LL, std::min<long long>(cap, (items_gu + 3) / 4));
  const int grid_dn = std::max(1, p.H / rt_dn);
  int rc;
  if (p.xq) {  // int8 activations: quantise x, gate/up, quantise the h rows, down
    if constexpr (QT == MOE_QTYPE_Q4_0 || QT == MOE_QTYPE_Q8_0) {
      if ((rc = launch_quant_act(ctx, x, (long long)p.T * p.H / kQK, p.xq, p.xs, p.xsum, s))) return rc;
      {
        KernelTimer timer(ctx, "ffn_gateup", s);
        dispatch_gateup<QT, true>(gu, p, x, grid_gu, s, nullptr);
      }
      if ((rc = check_launch("ffn_gateup_decode"))) return rc;
      if ((rc = launch_quant_act(ctx, p.hbuf, (long long)p.T * p.k * p.I / kQK, p.hq, p.hs, p.hsum, s))) return rc;
      {
        KernelTimer timer(ctx, "ffn_down", s);
        dispatch_down<QT, true>(dn, p, grid_dn, s);
      }
      return check_launch("ffn_down_decode");
    }
    return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "int8-activation decode: block type %d", QT);
  }
  // experts with many tokens of the batch on the matrix cores (fp32): their
  // gate/up and down kernels run on the context's side stream, beside the
  // GEMV gate/up of the other experts (they share no data), and are joined
  // before the down GEMV kernel, whose combine reads their y rows
  FfnParams q = p;
  const bool mix = mfma_decode_type(QT) && !route && p.T >= kMfmaMinBatch;
  const int grid_mx = 4 * ctx->num_cus;  // persistent: items in turn
  hipStream_t ms = s;
  if (mix) {
    q.mfma_min = kMfmaMinPairs;
    hipError_t e;
    if ((e = hipEventRecord(ctx->fork_ev, s)) != hipSuccess) return hip_error(e, "hipEventRecord(fork)");
    if ((e = hipStreamWaitEvent(ctx->side, ctx->fork_ev, 0)) != hipSuccess) return hip_error(e, "hipStreamWaitEvent(fork)");
    ms = ctx->side;
    if constexpr (mfma_decode_type(QT)) {
      KernelTimer timer(ctx, "ffn_gateup_mfma", ms);
      launch(ffn_gateup_mfma<QT>, grid_mx, kMfmaThreads, 0, ms, q, x);
    }
    if ((rc = check_launch("ffn_gateup_mfma"))) return rc;
    if constexpr (mfma_decode_type(QT)) {
      KernelTimer timer(ctx, "ffn_down_mfma", ms);
      launch(ffn_down_mfma<QT>, grid_mx, kMfmaThreads, 0, ms, q);
    }
    if ((rc = check_launch("ffn_down_mfma"))) return rc;
    if ((e = hipEventRecord(ctx->join_ev, ms)) != hipSuccess) return hip_error(e, "hipEventRecord(join)");
  }
  {
    KernelTimer timer(ctx, "ffn_gateup", s);
    dispatch_gateup<QT>(gu, q, x, grid_gu, s, route);
  }
  rc = check_launch("ffn_gateup_decode");
  if (rc) return rc;
  if (mix) {
    hipError_t e;
    if ((e = hipStreamWaitEvent(s, ctx->join_ev, 0)) != hipSuccess) return hip_error(e, "hipStreamWaitEvent(join)");
  }
  {
    KernelTimer timer(ctx, "ffn_down", s);
    dispatch_down<QT>(dn, q, grid_dn, s);
  }
  return check_launch("ffn_down_decode");
}

}  // namespace moe
