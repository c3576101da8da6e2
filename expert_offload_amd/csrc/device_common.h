// Device helpers shared by libmoe's kernels: block decoding from the packed
// slot layout, bf16 conversion and wavefront (64-lane) reductions.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16, round to nearest even (finite values).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// DPP lane moves inside a 16-lane row (no LDS crossbar).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16

// Wave-wide maximum / sum returned to every lane: four DPP steps reduce
// each 16-lane row, then the four row results are read as scalars.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = width / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, width);
  return v;
}

// Start of block `b` of one packed row, its scale d, offset m, fifth bits.
template <int QT>
__device__ __forceinline__ const uint8_t* block_quants(const uint8_t* row, int b) {
  return row + (size_t)(b >> 3) * group_bytes(QT) + (b & 7) * quant_bytes_per_block(QT);
}
// Q4_K's 6-bit scale and min codes of sub-block j from its 12 packed bytes
// sc: j < 4 in the low six bits of bytes j and j + 4; j >= 4 in the two
// nibbles of byte j + 4 with bits 4-5 in the top two bits of bytes j - 4 and j.
__device__ __forceinline__ int q4k_scale_code(const uint8_t* sc, int j) {
  return j < 4 ? (sc[j] & 63) : ((sc[j + 4] & 15) | ((sc[j - 4] >> 6) << 4));
}
__device__ __forceinline__ int q4k_min_code(const uint8_t* sc, int j) {
  return j < 4 ? (sc[j + 4] & 63) : ((sc[j + 4] >> 4) | ((sc[j] >> 6) << 4));
}

// K-quant sub-block b's scale d * scale_b and offset -dmin * min_b from one
// 16-byte load of the group's tail (12 scale bytes, d, dmin).
template <int QT>
__device__ __forceinline__ void q4k_block_dm(const uint8_t* row, int b, float& d, float& m) {
  static_assert(qtype_is_k(QT) && group_ksc_off(QT) % 16 == 0 && group_bytes(QT) % 16 == 0, "16-byte tail load");
  const uint8_t* g = row + (size_t)(b >> 3) * group_bytes(QT);
  const uint4 t = *reinterpret_cast<const uint4*>(g + group_ksc_off(QT));
  const uint32_t w[3] = {t.x, t.y, t.z};
  const int j = b & 7;
  auto byte = [&](int i) -> int { return (int)((w[i >> 2] >> (8 * (i & 3))) & 0xFFu); };
  const int sc = j < 4 ? (byte(j) & 63) : ((byte(j + 4) & 15) | ((byte(j - 4) >> 6) << 4));
  const int mn = j < 4 ? (byte(j + 4) & 63) : ((byte(j + 4) >> 4) | ((byte(j) >> 6) << 4));
  const float dd = __half2float(__ushort_as_half((unsigned short)(t.w & 0xFFFFu)));
  const float dm = __half2float(__ushort_as_half((unsigned short)(t.w >> 16)));
  d = dd * (float)sc;
  m = -(dm * (float)mn);
}

// K-quants: d * scale_j and -dmin * min_j are exact in fp32 (an 11-bit scale
// times a 6-bit code).
template <int QT>
__device__ __forceinline__ float block_scale(const uint8_t* row, int b) {
  const uint8_t* g = row + (size_t)(b >> 3) * group_bytes(QT);
  if constexpr (qtype_is_k(QT)) {
    const float d = __half2float(*reinterpret_cast<const __half*>(g + group_d_off(QT)));
    return d * (float)q4k_scale_code(g + group_ksc_off(QT), b & 7);
  } else {
    return __half2float(*reinterpret_cast<const __half*>(g + group_d_off(QT) + 2 * (b & 7)));
  }
}
template <int QT>
__device__ __forceinline__ float block_min(const uint8_t* row, int b) {
  if constexpr (qtype_is_k(QT)) {
    const uint8_t* g = row + (size_t)(b >> 3) * group_bytes(QT);
    const float dmin = __half2float(*reinterpret_cast<const __half*>(g + group_m_off(QT)));
    return -(dmin * (float)q4k_min_code(g + group_ksc_off(QT), b & 7));
  } else if constexpr (qtype_has_min(QT)) {
    const uint8_t* g = row + (size_t)(b >> 3) * group_bytes(QT);
    return __half2float(*reinterpret_cast<const __half*>(g + group_m_off(QT) + 2 * (b & 7)));
  } else {
    return 0.0f;
  }
}
template <int QT>
__device__ __forceinline__ uint32_t block_qh(const uint8_t* row, int b) {
  if constexpr (qtype_has_qh(QT)) {
    const uint8_t* g = row + (size_t)(b >> 3) * group_bytes(QT);
    return *reinterpret_cast<const uint32_t*>(g + group_qh_off(QT) + 4 * (b & 7));
  } else {
    return 0u;
  }
}

// Bits 0..3 of t (the fifth code bits of four consecutive elements) moved
// to bit 4 of each byte, to be or-ed into four nibble bytes.
__device__ __forceinline__ uint32_t spread_fifth_bits(uint32_t t) {
  return (((t & 0xFu) * 0x00204081u) & 0x01010101u) << 4;
}

// The 32 codes of block `b` as floats in logical element order: the signed
// code q (w = d * q) for Q8_0 (int8), Q4_0 (u - 8), Q5_0 (u - 16); the
// unsigned code u (w = d * u + m) for Q4_1, Q5_1, Q4_K and Q5_K.
template <int QT>
__device__ __forceinline__ void block_codes(const uint8_t* row, int b, float (&q)[32]) {
  const uint8_t* p = block_quants<QT>(row, b);
  if constexpr (QT == MOE_QTYPE_Q8_0) {
    const int4 v0 = *reinterpret_cast<const int4*>(p);
    const int4 v1 = *reinterpret_cast<const int4*>(p + 16);
    const int w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) q[4 * i + j] = (float)(int)(int8_t)(w[i] >> (8 * j));
    }
  } else {
    const int4 v = *reinterpret_cast<const int4*>(p);
    const uint32_t w[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
    const uint32_t qh = block_qh<QT>(row, b);
    constexpr int off = (int)qtype_code_off(QT);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
      if constexpr (qtype_has_qh(QT)) {
        lo |= spread_fifth_bits(qh >> (4 * i));
        hi |= spread_fifth_bits(qh >> (16 + 4 * i));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        q[4 * i + j] = (float)((int)((lo >> (8 * j)) & 0xFFu) - off);
        q[16 + 4 * i + j] = (float)((int)((hi >> (8 * j)) & 0xFFu) - off);
      }
    }
  }
}

}  // namespace moe
