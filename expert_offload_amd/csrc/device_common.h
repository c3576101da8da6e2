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

// Start of block `b` of one packed row, and its scale.
template <int QT>
__device__ __forceinline__ const uint8_t* block_quants(const uint8_t* row, int b) {
  return row + (size_t)(b >> 3) * group_bytes(QT) + (b & 7) * quant_bytes_per_block(QT);
}
template <int QT>
__device__ __forceinline__ float block_scale(const uint8_t* row, int b) {
  const uint8_t* g = row + (size_t)(b >> 3) * group_bytes(QT);
  const __half d = *reinterpret_cast<const __half*>(g + kGroupBlocks * quant_bytes_per_block(QT) + 2 * (b & 7));
  return __half2float(d);
}

// The 32 integer codes of block `b` as floats in logical element order:
// Q8_0 -> q (int8), Q4_0 -> q - 8.
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
    const int w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int byte = (w[i] >> (8 * j)) & 0xFF;
        q[4 * i + j] = (float)((byte & 0xF) - 8);
        q[16 + 4 * i + j] = (float)((byte >> 4) - 8);
      }
    }
  }
}

}  // namespace moe
