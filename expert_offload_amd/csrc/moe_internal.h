// Internal declarations shared by libmoe's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/moe.h"

struct moe_timing_rec {
  const char* kernel;
  hipEvent_t start, stop;
};

struct moe_ctx {
  int device;
  int num_cus;
  int* d_err;  // sticky device error word: 0, (expert id + 1), or INT_MIN
  bool timing = false;
  std::vector<moe_timing_rec> recs;
  std::vector<hipEvent_t> spare_events;
};

namespace moe {

// Brackets one kernel launch with HIP events on its stream while the
// context's timing is on (never inside a stream capture).
class KernelTimer {
 public:
  KernelTimer(moe_ctx* ctx, const char* kernel, hipStream_t s);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  moe_ctx* ctx_;
  hipStream_t s_;
  moe_timing_rec rec_{};
  bool on_ = false;
};

// ---------------------------------------------------------------- errors
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int hip_error(hipError_t e, const char* what);
int ensure_device(const moe_ctx* ctx);
int check_launch(const char* kernel);

// ------------------------------------------------------- device layout
// A matrix of `rows` x `cols` weights (cols % 256 == 0) is stored row by
// row; each row is cols/256 groups; a group holds 8 consecutive blocks:
// their quant bytes in ggml order, then their 8 fp16 scales.
constexpr int kQK = 32;            // weights per block
constexpr int kGroupBlocks = 8;    // blocks per group
constexpr int kGroupWeights = kQK * kGroupBlocks;  // 256

__host__ __device__ constexpr int quant_bytes_per_block(int qtype) {
  return qtype == MOE_QTYPE_Q8_0 ? 32 : 16;
}
__host__ __device__ constexpr int group_bytes(int qtype) {
  return kGroupBlocks * quant_bytes_per_block(qtype) + 2 * kGroupBlocks;
}
__host__ __device__ constexpr size_t row_bytes(int qtype, int cols) {
  return (size_t)(cols / kGroupWeights) * group_bytes(qtype);
}
__host__ __device__ constexpr size_t matrix_bytes(int qtype, int rows, int cols) {
  return (size_t)rows * row_bytes(qtype, cols);
}
// Per-slot offsets: gate [I][H], up [I][H], down [H][I].
__host__ __device__ constexpr size_t slot_gate_off(int, int, int) { return 0; }
__host__ __device__ constexpr size_t slot_up_off(int qtype, int H, int I) {
  return matrix_bytes(qtype, I, H);
}
__host__ __device__ constexpr size_t slot_down_off(int qtype, int H, int I) {
  return 2 * matrix_bytes(qtype, I, H);
}
__host__ __device__ constexpr size_t slot_bytes_of(int qtype, int H, int I) {
  return 2 * matrix_bytes(qtype, I, H) + matrix_bytes(qtype, H, I);
}

inline bool qtype_supported(int qtype) {
  return qtype == MOE_QTYPE_Q8_0 || qtype == MOE_QTYPE_Q4_0;
}
inline const char* qtype_name(int qtype) {
  return qtype == MOE_QTYPE_Q8_0 ? "Q8_0" : qtype == MOE_QTYPE_Q4_0 ? "Q4_0" : "?";
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;

}  // namespace moe
