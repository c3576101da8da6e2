// Expert-FFN kernels on the vector ALUs (fp32 activations or bf16
// activations widened to fp32, fp32 accumulation) for the shapes the tuned
// kernels do not take: decode batches of more than 1024 (token, expert)
// pairs and prefill with fp32 activations.
//
// Work is split into (active expert, row tile) items; each item streams its
// rows' quant blocks once per group of up to 8 of the expert's pairs.
#include <algorithm>
#include <cmath>

#include "device_common.h"
#include "ffn.h"

namespace moe {

namespace {

template <typename XT>
__device__ __forceinline__ void load_x32(const XT* xrow, int col, float (&xv)[32]) {
  if constexpr (sizeof(XT) == 4) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(xrow + col + 4 * i);
      xv[4 * i] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(xrow + col + 8 * i);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[8 * i + 2 * j] = bf16_to_f32(w[j] & 0xFFFF);
        xv[8 * i + 2 * j + 1] = bf16_to_f32(w[j] >> 16);
      }
    }
  }
}

}  // namespace

// Gate/up + SwiGLU.  An item is (active expert, 8 intermediate indices);
// thread row r < 8 computes gate row i = 8*tile + r, r >= 8 the up row;
// 16 lanes share a row and stride over its blocks.
template <int QT, typename XT>
__global__ __launch_bounds__(256) void ffn_gateup_valu(FfnParams p, const XT* __restrict__ x) {
  __shared__ float s_gu[16][8];
  const int r = threadIdx.x >> 4, l16 = threadIdx.x & 15;
  const int n_tiles = p.I / 8;
  const int items = p.active[0] * n_tiles;
  const int nblk = p.H / kQK;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int a = item / n_tiles, tile = item - a * n_tiles;
    const int e = p.active[1 + a];
    if (p.mask && !p.mask[e]) continue;
    const int slot = p.slot_table[e];
    const int pbeg = p.offsets[e], n_e = p.offsets[e + 1] - pbeg;
    if (slot < 0 || slot >= p.n_slots) {
      if (threadIdx.x == 0) atomicCAS(p.err, 0, e + 1);
      for (int s = threadIdx.x; s < n_e * 8; s += 256)
        p.hbuf[(size_t)(pbeg + s / 8) * p.I + tile * 8 + (s & 7)] = NAN;
      continue;
    }
    const uint8_t* base = p.pool + (size_t)slot * p.slot_bytes;
    const size_t moff = r < 8 ? slot_gate_off(QT, p.H, p.I) : slot_up_off(QT, p.H, p.I);
    const uint8_t* row = base + moff + (size_t)(tile * 8 + (r & 7)) * row_bytes(QT, p.H);
    for (int tg = 0; tg < n_e; tg += 8) {
      const int nt = min(8, n_e - tg);
      const XT* xr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tok = j < nt ? p.sorted_pairs[pbeg + tg + j] / p.k : 0;
        xr[j] = x + (size_t)tok * p.H;
      }
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int b = l16; b < nblk; b += 16) {
        float q[32];
        block_codes<QT>(row, b, q);
        const float d = block_scale<QT>(row, b), m = block_min<QT>(row, b);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j < nt) {
            float xv[32];
            load_x32(xr[j], b * kQK, xv);
            float dot = 0.0f, sx = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) dot = fmaf(q[i], xv[i], dot);
            if constexpr (qtype_has_min(QT)) {
#pragma unroll
              for (int i = 0; i < 32; ++i) sx += xv[i];
              acc[j] = fmaf(m, sx, acc[j]);
            }
            acc[j] = fmaf(d, dot, acc[j]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = group_sum<16>(acc[j]);
      if (l16 == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) s_gu[r][j] = acc[j];
      }
      __syncthreads();
      if (threadIdx.x < 64) {
        const int ii = threadIdx.x & 7, j = threadIdx.x >> 3;
        if (j < nt) {
          const float g = s_gu[ii][j], u = s_gu[8 + ii][j];
          p.hbuf[(size_t)(pbeg + tg + j) * p.I + tile * 8 + ii] = g / (1.0f + expf(-g)) * u;
        }
      }
      __syncthreads();
    }
  }
}

// Down projection.  An item is (active expert, 16 output rows); 16 lanes per
// row stride over the row's blocks; inputs are the expert's h rows.
template <int QT>
__global__ __launch_bounds__(256) void ffn_down_valu(FfnParams p) {
  const int r = threadIdx.x >> 4, l16 = threadIdx.x & 15;
  const int n_tiles = p.H / 16;
  const int items = p.active[0] * n_tiles;
  const int nblk = p.I / kQK;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int a = item / n_tiles, tile = item - a * n_tiles;
    const int e = p.active[1 + a];
    if (p.mask && !p.mask[e]) continue;
    const int slot = p.slot_table[e];
    const int pbeg = p.offsets[e], n_e = p.offsets[e + 1] - pbeg;
    const int orow = tile * 16 + r;
    if (slot < 0 || slot >= p.n_slots) {
      if (l16 == 0)
        for (int j = 0; j < n_e; ++j) p.y[(size_t)p.sorted_pairs[pbeg + j] * p.H + orow] = NAN;
      continue;
    }
    const uint8_t* row = p.pool + (size_t)slot * p.slot_bytes + slot_down_off(QT, p.H, p.I) +
                         (size_t)orow * row_bytes(QT, p.I);
    for (int tg = 0; tg < n_e; tg += 8) {
      const int nt = min(8, n_e - tg);
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int b = l16; b < nblk; b += 16) {
        float q[32];
        block_codes<QT>(row, b, q);
        const float d = block_scale<QT>(row, b), m = block_min<QT>(row, b);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j < nt) {
            float hv[32];
            load_x32(p.hbuf + (size_t)(pbeg + tg + j) * p.I, b * kQK, hv);
            float dot = 0.0f, sx = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) dot = fmaf(q[i], hv[i], dot);
            if constexpr (qtype_has_min(QT)) {
#pragma unroll
              for (int i = 0; i < 32; ++i) sx += hv[i];
              acc[j] = fmaf(m, sx, acc[j]);
            }
            acc[j] = fmaf(d, dot, acc[j]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = group_sum<16>(acc[j]);
      if (l16 == 0) {
        for (int j = 0; j < nt; ++j) p.y[(size_t)p.sorted_pairs[pbeg + tg + j] * p.H + orow] = acc[j];
      }
    }
  }
}

template <int QT>
static int launch_ffn_valu_t(moe_ctx* ctx, const FfnParams& p, const void* x, int x_dtype, hipStream_t s) {
  const int grid_cap = 8 * ctx->num_cus;
  const int max_active = std::min(p.E, p.T * p.k);
  const int g1 = std::max(1, std::min(grid_cap, max_active * (p.I / 8)));
  const int g2 = std::max(1, std::min(grid_cap, max_active * (p.H / 16)));
  {
    KernelTimer timer(ctx, "ffn_gateup", s);
    if (x_dtype == MOE_DTYPE_F32) launch(ffn_gateup_valu<QT, float>, g1, 256, 0, s, p, (const float*)x);
    else launch(ffn_gateup_valu<QT, uint16_t>, g1, 256, 0, s, p, (const uint16_t*)x);
  }
  int rc = check_launch("ffn_gateup_valu");
  if (rc) return rc;
  {
    KernelTimer timer(ctx, "ffn_down", s);
    launch(ffn_down_valu<QT>, g2, 256, 0, s, p);
  }
  return check_launch("ffn_down_valu");
}

int launch_ffn_valu(moe_ctx* ctx, const FfnParams& p, const void* x, int x_dtype, hipStream_t s) {
  switch (p.qtype) {
    case MOE_QTYPE_Q8_0: return launch_ffn_valu_t<MOE_QTYPE_Q8_0>(ctx, p, x, x_dtype, s);
    case MOE_QTYPE_Q4_0: return launch_ffn_valu_t<MOE_QTYPE_Q4_0>(ctx, p, x, x_dtype, s);
    case MOE_QTYPE_Q4_1: return launch_ffn_valu_t<MOE_QTYPE_Q4_1>(ctx, p, x, x_dtype, s);
    case MOE_QTYPE_Q5_0: return launch_ffn_valu_t<MOE_QTYPE_Q5_0>(ctx, p, x, x_dtype, s);
    case MOE_QTYPE_Q5_1: return launch_ffn_valu_t<MOE_QTYPE_Q5_1>(ctx, p, x, x_dtype, s);
    case MOE_QTYPE_Q4_K: return launch_ffn_valu_t<MOE_QTYPE_Q4_K>(ctx, p, x, x_dtype, s);
    case MOE_QTYPE_Q5_K: return launch_ffn_valu_t<MOE_QTYPE_Q5_K>(ctx, p, x, x_dtype, s);
    default: return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "expert FFN: block type %d", p.qtype);
  }
}

}  // namespace moe
