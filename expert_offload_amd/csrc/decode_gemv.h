// Building blocks of the decode dequant-GEMV kernels: raw block loads,
// the block dot product, the transposed butterfly that folds
// per-lane row sums, activation staging, and the shape rules (rows per lane
// within a register budget).
//
// GEMV layout.  A wavefront owns RW = (64 / LPR) * RPL weight rows: lanes
// form 64/LPR groups of LPR lanes, each group covers RPL rows, and every
// lane owns the same BPL column blocks of all its rows.  The lane issues
// all of its rows' 16-byte quant loads before any arithmetic (enough bytes
// in flight to cover HBM latency), reuses each activation block for RPL
// rows, and the RPL partial sums are folded across the LPR lanes with a
// transposed butterfly (RPL - 1 + log2(LPR / RPL) shuffles instead of
// RPL * log2(LPR)).
//
// Block arithmetic.  With u the unsigned code (Q8_0: q + 128 after
// flipping the sign bit), sum_k w_k x_k = d * (sum_k u_k x_k - OFF * sum_k
// x_k), OFF = 128 (Q8_0), 8 (Q4_0) or 16 (Q5_0); Q4_1 / Q5_1: d * sum_k
// u_k x_k + m * sum_k x_k.  sum_k x_k is formed once per block and token
// and shared by the lane's RPL rows.  The down kernel takes Q8_0 as
// d * sum_k q_k x_k instead, each signed byte converted in one
// instruction (RowTile's SGN).
#pragma once

#include "device_common.h"

namespace moe {

// --------------------------------------------------------------- helpers
template <int QT>
struct QTraits {
  static constexpr int kWords = QT == MOE_QTYPE_Q8_0 ? 8 : 4;  // 32 or 16 bytes of codes
  static constexpr bool kQh = qtype_has_qh(QT);               // a word of fifth bits
  static constexpr bool kMin = qtype_has_min(QT);             // w = d*u + m
  static constexpr float kOff = qtype_code_off(QT);           // else w = d*(u - kOff)
  static constexpr int kRegs = kWords + (kQh ? 1 : 0);
};

template <int QT>
__device__ __forceinline__ void load_block_raw(const uint8_t* row, int b, uint32_t (&w)[QTraits<QT>::kWords],
                                               float& d) {
  const uint8_t* q = block_quants<QT>(row, b);
  const uint4 v0 = *reinterpret_cast<const uint4*>(q);
  w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
  if constexpr (QT == MOE_QTYPE_Q8_0) {
    const uint4 v1 = *reinterpret_cast<const uint4*>(q + 16);
    w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
  }
  d = block_scale<QT>(row, b);
}

__device__ __forceinline__ void load_f32x32(const float* p, float (&xv)[32]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(p + 4 * i);
    xv[4 * i] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
  }
}

__device__ __forceinline__ float sum32(const float (&xv)[32]) {
  float a = 0.0f, b = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i += 2) {
    a += xv[i];
    b += xv[i + 1];
  }
  return a + b;
}

// Transposed butterfly over aligned groups of LPR lanes: on entry lane l
// holds partial sums v[0..N) of N rows; on exit v[0] of every lane holds the
// full sum of row (l % LPR) / (LPR / N) of its group.
template <int OFF, int N, int M>
__device__ __forceinline__ void fold_rows(float (&v)[M], int lane) {
  if constexpr (OFF >= 1) {
    if constexpr (N > 1) {
      const bool hi = (lane & OFF) != 0;
#pragma unroll
      for (int r = 0; r < N / 2; ++r) {
        const float keep = hi ? v[r + N / 2] : v[r];
        const float send = hi ? v[r] : v[r + N / 2];
        v[r] = keep + __shfl_xor(send, OFF, kWave);
      }
      fold_rows<OFF / 2, N / 2, M>(v, lane);
    } else {
      v[0] += __shfl_xor(v[0], OFF, kWave);
      fold_rows<OFF / 2, 1, M>(v, lane);
    }
  }
}

// Rows of one lane's GEMV: RPL rows x BPL blocks of raw codes, fifth bits,
// scales and offsets (the last two only for the types that have them).
// SGN (Q8_0 only): convert the signed codes directly instead of adding the
// offset back; the down kernel measured faster so, the gate/up kernel
// slower (the two forms round differently, each is used by one kernel).
template <int QT, int LPR, int BPL, int RPL, bool SGN = false>
struct RowTile {
  using Q = QTraits<QT>;
  static constexpr bool kSigned = SGN && QT == MOE_QTYPE_Q8_0;
  uint32_t w[RPL][BPL][Q::kWords];
  uint32_t qh[RPL][BPL];
  float d[RPL][BPL];
  float m[RPL][BPL];

  __device__ __forceinline__ void load(const uint8_t* const (&rows)[RPL], int lg) {
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        if constexpr (qtype_is_k(QT)) {  // codes, then scale and offset from one load
          const uint4 v = *reinterpret_cast<const uint4*>(block_quants<QT>(rows[r], lg + LPR * i));
          w[r][i][0] = v.x; w[r][i][1] = v.y; w[r][i][2] = v.z; w[r][i][3] = v.w;
          q4k_block_dm<QT>(rows[r], lg + LPR * i, d[r][i], m[r][i]);
          if constexpr (Q::kQh) qh[r][i] = block_qh<QT>(rows[r], lg + LPR * i);
          continue;
        }
        load_block_raw<QT>(rows[r], lg + LPR * i, w[r][i], d[r][i]);
        if constexpr (Q::kQh) qh[r][i] = block_qh<QT>(rows[r], lg + LPR * i);
        if constexpr (Q::kMin) m[r][i] = block_min<QT>(rows[r], lg + LPR * i);
      }
  }

  // acc[r] = sum over the lane's blocks of d * (u . x - OFF * sum x) (or
  // d * (q . x) with SGN), or d * (u . x) + m * sum x for the types with
  // an offset m, with the lane's
  // activation blocks already in xv.  Rows are finished one at a time in
  // load order, so the wait before row r covers only the loads up to row r
  // and row r's math overlaps the later rows' transfers.  Each row's codes
  // pass through an empty asm right before use so the compiler widens them
  // here, inside the token loop, instead of keeping RPL*BPL*32 widened
  // floats live; four partial sums per row break the FMA dependency chain.
  __device__ __forceinline__ void dot(const float (&xv)[BPL][32], float (&acc)[RPL]) {
    float sx[BPL];
#pragma unroll
    for (int i = 0; i < BPL; ++i) sx[i] = block_sx(xv[i]);
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      acc[r] = 0.0f;
#pragma unroll
      for (int i = 0; i < BPL; ++i) acc[r] = block_dot(r, i, xv[i], sx[i], acc[r]);
    }
  }

  // The same sums for one row, with each activation block read from a
  // swizzled LDS row (see hswz) right before its use, so only 32
  // activations are live at a time; bit-identical to dot.
  __device__ __forceinline__ void dot_lds_swz(const float* row, int lg, float (&acc)[RPL]) {
    static_assert(RPL == 1, "one row per lane");
    acc[0] = 0.0f;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      float xb[32];
      const int b = lg + LPR * i;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(row + (b << 5) + (((j + b) & 7) << 2));
        xb[4 * j] = v.x; xb[4 * j + 1] = v.y; xb[4 * j + 2] = v.z; xb[4 * j + 3] = v.w;
      }
      acc[0] = block_dot(0, i, xb, block_sx(xb), acc[0]);
    }
  }

  // int8 activations (MOE_MODE_DECODE_Q8A): acc[r] = sum over the lane's
  // blocks of (d * s) * (integer sum of weight code x activation code), the
  // integer sums by 4-way int8 dot products (Q4_0: codes u - 8 as
  // sum(u q) - 8 sum(q); Q8_0: the signed codes as stored).
  template <typename A>
  __device__ __forceinline__ void dot_q8(const A& a, float (&acc)[RPL]) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      acc[r] = 0.0f;
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
#pragma unroll
        for (int q = 0; q < Q::kWords; ++q) asm volatile("" : "+v"(w[r][i][q]));
        int isum = 0;
        if constexpr (QT == MOE_QTYPE_Q8_0) {
#pragma unroll
          for (int q = 0; q < 8; ++q) isum = __builtin_amdgcn_sdot4((int)w[r][i][q], (int)a.q[i][q], isum, false);
        } else {
          static_assert(QT == MOE_QTYPE_Q4_0, "int8 activations take Q4_0 and Q8_0 codes");
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            isum = __builtin_amdgcn_sdot4((int)(w[r][i][q] & 0x0F0F0F0Fu), (int)a.q[i][q], isum, false);
            isum = __builtin_amdgcn_sdot4((int)((w[r][i][q] >> 4) & 0x0F0F0F0Fu), (int)a.q[i][4 + q], isum, false);
          }
          isum -= 8 * a.sum[i];
        }
        acc[r] = fmaf(d[r][i] * a.s[i], (float)isum, acc[r]);
      }
    }
  }

  __device__ __forceinline__ static float block_sx(const float (&x)[32]) {
    if constexpr (kSigned) return 0.0f;  // signed codes: no offset term
    else return Q::kMin ? sum32(x) : sum32(x) * Q::kOff;
  }

  // acc + this lane's block i of row r against x: d * (u . x - sx) or
  // d * (u . x) + m * sx, with sx from block_sx.
  __device__ __forceinline__ float block_dot(int r, int i, const float (&x)[32], float sx, float acc) {
#pragma unroll
    for (int q = 0; q < Q::kWords; ++q) asm volatile("" : "+v"(w[r][i][q]));
    float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (kSigned) {
      // each signed byte converts in one instruction (byte-select sign
      // extension), so no offset is folded in
#pragma unroll
      for (int q = 0; q < 8; ++q) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          part[j] = fmaf((float)(int8_t)(w[r][i][q] >> (8 * j)), x[4 * q + j], part[j]);
      }
    } else if constexpr (QT == MOE_QTYPE_Q8_0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t u = w[r][i][q] ^ 0x80808080u;  // q + 128 in every byte
#pragma unroll
        for (int j = 0; j < 4; ++j) part[j] = fmaf((float)((u >> (8 * j)) & 0xFFu), x[4 * q + j], part[j]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t lo = w[r][i][q] & 0x0F0F0F0Fu, hi = (w[r][i][q] >> 4) & 0x0F0F0F0Fu;
        if constexpr (Q::kQh) {
          lo |= spread_fifth_bits(qh[r][i] >> (4 * q));
          hi |= spread_fifth_bits(qh[r][i] >> (16 + 4 * q));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          part[j] = fmaf((float)((lo >> (8 * j)) & 0xFFu), x[4 * q + j], part[j]);
          part[j] = fmaf((float)((hi >> (8 * j)) & 0xFFu), x[16 + 4 * q + j], part[j]);
        }
      }
    }
    const float su = (part[0] + part[1]) + (part[2] + part[3]);
    if constexpr (Q::kMin) return fmaf(d[r][i], su, fmaf(m[r][i], sx, acc));
    else return fmaf(d[r][i], su - sx, acc);
  }
};

// The lane's BPL int8 activation blocks of one row (MOE_MODE_DECODE_Q8A):
// 32 codes as 8 words (word q = elements 4q .. 4q+3), the block scale and
// the sum of its codes.
template <int LPR, int BPL>
struct ActQ8 {
  uint32_t q[BPL][8];
  float s[BPL];
  int sum[BPL];
  __device__ __forceinline__ void load(const int8_t* codes, const float* scales, const int* sums, int lg) {
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int b = lg + LPR * i;
      const uint4 v0 = *reinterpret_cast<const uint4*>(codes + (size_t)b * kQK);
      const uint4 v1 = *reinterpret_cast<const uint4*>(codes + (size_t)b * kQK + 16);
      q[i][0] = v0.x; q[i][1] = v0.y; q[i][2] = v0.z; q[i][3] = v0.w;
      q[i][4] = v1.x; q[i][5] = v1.y; q[i][6] = v1.z; q[i][7] = v1.w;
      s[i] = scales[b];
      sum[i] = sums[b];
    }
  }
};

// The lane's BPL activation blocks of one token row.
template <int LPR, int BPL>
__device__ __forceinline__ void load_act(const float* act, int lg, float (&xv)[BPL][32]) {
#pragma unroll
  for (int i = 0; i < BPL; ++i) load_f32x32(act + (size_t)(lg + LPR * i) * kQK, xv[i]);
}


constexpr int kDownWaves = 8;
constexpr int kDownLdsFloats = 2048;    // y tile kept in LDS for the combine when T*k*RW fits
constexpr int kDownStageFloats = 1024;  // per-wave staging of one h row when I fits
constexpr int kStageVec = kDownStageFloats / (4 * kWave);  // float4 per lane

// Staged h rows are swizzled in LDS: within each 32-float block b, float4 j
// sits in slot (j + b) mod 8.  The lanes of a row group read blocks lg +
// LPR*i at the same j; plain, those are 128 B apart and hit the same banks,
// swizzled they fall in 8 different 16-byte slots.
__device__ __forceinline__ int hswz(int c) {  // float index c (a multiple of 4) -> LDS position
  const int b = c >> 5, j = (c >> 2) & 7;
  return (b << 5) | (((j + b) & 7) << 2);
}

// The lane's BPL activation blocks from a swizzled LDS row.
template <int LPR, int BPL>
__device__ __forceinline__ void load_act_swz(const float* row, int lg, float (&xv)[BPL][32]) {
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = lg + LPR * i;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(row + (b << 5) + (((j + b) & 7) << 2));
      xv[i][4 * j] = v.x; xv[i][4 * j + 1] = v.y; xv[i][4 * j + 2] = v.z; xv[i][4 * j + 3] = v.w;
    }
  }
}

// One h row (I <= kDownStageFloats floats) in registers, on its way to LDS
// (stored swizzled, see hswz).
struct HRowRegs {
  float4 v[kStageVec];
  // Lanes past the row end re-read its last 4 floats (in bounds) and skip
  // the store, so every element is written unconditionally here.
  __device__ __forceinline__ void load(const float* src, int I, int lane) {
#pragma unroll
    for (int i = 0; i < kStageVec; ++i) {
      const int c = min((lane + kWave * i) * 4, I - 4);
      v[i] = *reinterpret_cast<const float4*>(src + c);
    }
  }
  __device__ __forceinline__ void store(float* dst, int I, int lane) const {
#pragma unroll
    for (int i = 0; i < kStageVec; ++i) {
      const int c = (lane + kWave * i) * 4;
      if (c < I) *reinterpret_cast<float4*>(dst + hswz(c)) = v[i];
    }
  }
};

// ----------------------------------------------------------- shape rules
template <int QT, int BPL>
constexpr int rows_per_lane() {
  constexpr int budget = 64 / (BPL * QTraits<QT>::kRegs);  // <= 64 registers of raw codes
  return budget >= 8 ? 8 : budget >= 4 ? 4 : budget >= 2 ? 2 : 1;
}
// Down tiles aim at 8 rows (H/8 workgroups): RPL = 8 / (64 / LPR) within
// the register budget.
template <int QT, int LPR, int BPL>
constexpr int down_rows_per_lane() {
  constexpr int want = 8 / (kWave / LPR) > 0 ? 8 / (kWave / LPR) : 1;
  constexpr int budget = rows_per_lane<QT, BPL>();
  return want < budget ? want : budget;
}

}  // namespace moe
