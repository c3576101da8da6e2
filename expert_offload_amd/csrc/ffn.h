// Expert-FFN launch parameters shared by the kernel families.
#pragma once

#include "moe_internal.h"

namespace moe {

struct FfnParams {
  const uint8_t* pool;
  size_t slot_bytes;
  int n_slots;
  int qtype;
  int H, I, T, k, E;
  const int32_t* slot_table;
  const int32_t* offsets;
  const int32_t* sorted_pairs;
  const int32_t* active;
  const int32_t* mask;
  float* y;     // [T*k][H] fp32, pair order
  float* hbuf;  // [T*k][I] fp32, grouped (sorted) order
  int* err;
};

int launch_ffn_valu(const FfnParams& p, const void* x, int x_dtype, int grid_cap, hipStream_t s);

}  // namespace moe
