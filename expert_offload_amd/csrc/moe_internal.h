// Internal declarations shared by libmoe's translation units.
#pragma once

#include <hip/hip_ext.h>
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
  void* d_scratch = nullptr;  // this device's static scratch array (moe_decode_layer_static)
  bool timing = false;
  std::vector<moe_timing_rec> recs;
  std::vector<hipEvent_t> spare_events;
  // a second stream (default priority) on which kernels independent of the
  // caller's stream's next ones run, forked and joined with these events
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
};

namespace moe {

// Times the one kernel launched through launch() while it is alive, if the
// context's timing is on and the stream is not being captured.  The start
// and stop events ride on the launch itself (hipExtLaunchKernel), so their
// elapsed time is the kernel's own execution, not the gap between markers.
class KernelTimer {
 public:
  KernelTimer(moe_ctx* ctx, const char* kernel, hipStream_t s);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

  // The innermost timer alive on this thread that still waits for its launch.
  static KernelTimer* armed();
  hipEvent_t start_event() const { return rec_.start; }
  hipEvent_t stop_event() const { return rec_.stop; }
  void launched() { launched_ = true; }

 private:
  moe_ctx* ctx_;
  KernelTimer* prev_ = nullptr;
  moe_timing_rec rec_{};
  bool on_ = false, launched_ = false;
};

// Launch `kern` on `s`, timed by the armed KernelTimer if there is one.
template <typename... P, typename... A>
inline void launch(void (*kern)(P...), dim3 grid, dim3 block, uint32_t lds, hipStream_t s, A... args) {
  if (KernelTimer* t = KernelTimer::armed()) {
    hipExtLaunchKernelGGL(kern, grid, block, lds, s, t->start_event(), t->stop_event(), 0u, static_cast<P>(args)...);
    t->launched();
  } else {
    kern<<<grid, block, lds, s>>>(static_cast<P>(args)...);
  }
}

// ---------------------------------------------------------------- errors
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int hip_error(hipError_t e, const char* what);
int ensure_device(const moe_ctx* ctx);
// Device address of the static scratch array on `device` (current), looked
// up once per device.
int static_scratch_init(int device, void** out);
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
__host__ __device__ constexpr bool qtype_has_min(int qtype) {  // w = d*q + m
  return qtype == MOE_QTYPE_Q4_1 || qtype == MOE_QTYPE_Q5_1 || qtype == MOE_QTYPE_Q4_K || qtype == MOE_QTYPE_Q5_K;
}
// Q4_K, Q5_K: one super-block of 256 weights per group; its 8 sub-blocks'
// scales d * scale_j and offsets -dmin * min_j come from the super-block's
// fp16 d, dmin and 6-bit codes.
__host__ __device__ constexpr bool qtype_is_k(int qtype) {
  return qtype == MOE_QTYPE_Q4_K || qtype == MOE_QTYPE_Q5_K;
}
__host__ __device__ constexpr bool qtype_has_qh(int qtype) {  // fifth code bits
  return qtype == MOE_QTYPE_Q5_0 || qtype == MOE_QTYPE_Q5_1 || qtype == MOE_QTYPE_Q5_K;
}
// ggml block bytes: fp16 d, [fp16 m], [4 B fifth bits], quant bytes.
__host__ __device__ constexpr int ggml_block_bytes(int qtype) {
  return 2 + (qtype_has_min(qtype) ? 2 : 0) + (qtype_has_qh(qtype) ? 4 : 0) + quant_bytes_per_block(qtype);
}
// K-quant super-blocks: Q4_K 144 bytes (fp16 d, fp16 dmin, 12 bytes of
// 6-bit scales and mins, 128 bytes of nibbles); Q5_K 176 (the same and 32
// bytes of fifth bits).  A group holds the same bytes.
__host__ __device__ constexpr int k_superblock_bytes(int qtype) {
  return 4 + 12 + kGroupWeights / 2 + (qtype_has_qh(qtype) ? kGroupWeights / 8 : 0);
}
__host__ __device__ constexpr int group_bytes(int qtype) {
  return qtype_is_k(qtype) ? k_superblock_bytes(qtype) : kGroupBlocks * ggml_block_bytes(qtype);
}
// Offsets inside a group: quant bytes at 0, then fifth-bit words, scales d,
// offsets m.  K-quants: quant bytes (per sub-block, nibble order of the
// 32-weight types), [fifth-bit words,] the 12 scale bytes, d, dmin.
__host__ __device__ constexpr int group_qh_off(int qtype) { return kGroupBlocks * quant_bytes_per_block(qtype); }
__host__ __device__ constexpr int group_ksc_off(int qtype) {
  return group_qh_off(qtype) + (qtype_has_qh(qtype) ? 4 * kGroupBlocks : 0);
}
__host__ __device__ constexpr int group_d_off(int qtype) {
  return qtype_is_k(qtype) ? group_ksc_off(qtype) + 12
                           : group_qh_off(qtype) + (qtype_has_qh(qtype) ? 4 * kGroupBlocks : 0);
}
__host__ __device__ constexpr int group_m_off(int qtype) {
  return group_d_off(qtype) + (qtype_is_k(qtype) ? 2 : 2 * kGroupBlocks);
}
// The stored code u (Q8_0: q + 128; 4-bit: the nibble; 5-bit: nibble + 16 *
// fifth bit) maps to w = d*u - OFF*d, or d*u + m for the types with m.
__host__ __device__ constexpr float qtype_code_off(int qtype) {
  return qtype == MOE_QTYPE_Q8_0 ? 128.0f : qtype == MOE_QTYPE_Q4_0 ? 8.0f : qtype == MOE_QTYPE_Q5_0 ? 16.0f : 0.0f;
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
  return qtype == MOE_QTYPE_Q8_0 || qtype == MOE_QTYPE_Q4_0 || qtype == MOE_QTYPE_Q4_1 || qtype == MOE_QTYPE_Q5_0 ||
         qtype == MOE_QTYPE_Q5_1 || qtype == MOE_QTYPE_Q4_K || qtype == MOE_QTYPE_Q5_K;
}
inline const char* qtype_name(int qtype) {
  switch (qtype) {
    case MOE_QTYPE_Q8_0: return "Q8_0";
    case MOE_QTYPE_Q4_0: return "Q4_0";
    case MOE_QTYPE_Q4_1: return "Q4_1";
    case MOE_QTYPE_Q5_0: return "Q5_0";
    case MOE_QTYPE_Q5_1: return "Q5_1";
    case MOE_QTYPE_Q4_K: return "Q4_K";
    case MOE_QTYPE_Q5_K: return "Q5_K";
    default: return "?";
  }
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;

// ------------------------------------------------------------ host executor
// The expert FFN on the host cores (host_ffn.cpp): n_exp experts, expert i
// in the slot at slots[i] (host memory), over the tokens tok[i][0..cnt[i])
// of x [*][H]; the output of its j-th token goes to row yrow[i][j] of
// y [*][H].  h: scratch of sum(cnt) * I floats.  Calls are serialised.
int host_experts_ffn(int qtype, int H, int I, int n_exp, const uint8_t* const* slots, const int* cnt,
                     const int* const* tok, const int* const* yrow, const float* x, float* y, float* h,
                     int threads, bool vector);
int default_host_threads();

}  // namespace moe
