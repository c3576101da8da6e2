// Host-side parts of libmoe: error reporting, the context, the block-type
// table and the ggml -> device layout packer.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "moe_internal.h"

namespace moe {

static thread_local std::string g_err;

int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

void clear_error() { g_err.clear(); }

int hip_error(hipError_t e, const char* what) {
  return set_error(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int ensure_device(const moe_ctx* ctx) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_error(e, "hipGetDevice");
  if (cur != ctx->device) {
    e = hipSetDevice(ctx->device);
    if (e != hipSuccess) return hip_error(e, "hipSetDevice");
  }
  return MOE_OK;
}

int check_launch(const char* kernel) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_error(e, kernel);
  return MOE_OK;
}

static hipEvent_t take_event(moe_ctx* ctx) {
  if (!ctx->spare_events.empty()) {
    hipEvent_t e = ctx->spare_events.back();
    ctx->spare_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

static thread_local KernelTimer* g_timer = nullptr;

KernelTimer::KernelTimer(moe_ctx* ctx, const char* kernel, hipStream_t s) : ctx_(ctx) {
  if (!ctx || !ctx->timing) return;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess || st != hipStreamCaptureStatusNone) return;
  rec_.kernel = kernel;
  rec_.start = take_event(ctx);
  rec_.stop = take_event(ctx);
  if (!rec_.start || !rec_.stop) {
    if (rec_.start) ctx->spare_events.push_back(rec_.start);
    if (rec_.stop) ctx->spare_events.push_back(rec_.stop);
    return;
  }
  on_ = true;
  prev_ = g_timer;
  g_timer = this;
}

KernelTimer::~KernelTimer() {
  if (!on_) return;
  g_timer = prev_;
  if (launched_) {
    ctx_->recs.push_back(rec_);
  } else {
    ctx_->spare_events.push_back(rec_.start);
    ctx_->spare_events.push_back(rec_.stop);
  }
}

KernelTimer* KernelTimer::armed() {
  return g_timer && !g_timer->launched_ ? g_timer : nullptr;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_ctx_create(int device, moe_ctx** out) {
  clear_error();
  if (!out) return set_error(MOE_ERR_INVALID_ARG, "moe_ctx_create: out is NULL");
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess) return hip_error(e, "hipGetDeviceCount");
  if (device < 0 || device >= n)
    return set_error(MOE_ERR_INVALID_ARG, "moe_ctx_create: device %d not in [0, %d)", device, n);
  if ((e = hipSetDevice(device)) != hipSuccess) return hip_error(e, "hipSetDevice");
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_error(e, "hipDeviceGetAttribute");
  moe_ctx* c = new moe_ctx;
  c->device = device;
  c->num_cus = cus;
  c->d_err = nullptr;
  if ((e = hipMalloc(&c->d_err, sizeof(int))) != hipSuccess) {
    delete c;
    return hip_error(e, "hipMalloc(error word)");
  }
  if ((e = hipMemset(c->d_err, 0, sizeof(int))) != hipSuccess) {
    (void)hipFree(c->d_err);
    delete c;
    return hip_error(e, "hipMemset(error word)");
  }
  int rc = static_scratch_init(device, &c->d_scratch);
  if (rc) {
    (void)hipFree(c->d_err);
    delete c;
    return rc;
  }
  if ((e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&c->fork_ev, hipEventDisableTiming)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&c->join_ev, hipEventDisableTiming)) != hipSuccess) {
    if (c->join_ev) (void)hipEventDestroy(c->join_ev);
    if (c->fork_ev) (void)hipEventDestroy(c->fork_ev);
    if (c->side) (void)hipStreamDestroy(c->side);
    (void)hipFree(c->d_err);
    delete c;
    return hip_error(e, "moe_ctx_create: side stream and events");
  }
  *out = c;
  return MOE_OK;
}

int moe_ctx_set_timing(moe_ctx* ctx, int enable) {
  clear_error();
  if (!ctx) return set_error(MOE_ERR_INVALID_ARG, "moe_ctx_set_timing: ctx is NULL");
  for (auto& r : ctx->recs) {
    ctx->spare_events.push_back(r.start);
    ctx->spare_events.push_back(r.stop);
  }
  ctx->recs.clear();
  ctx->timing = enable != 0;
  return MOE_OK;
}

int moe_ctx_kernel_time(moe_ctx* ctx, const char* kernel, int* count, double* total_ms) {
  clear_error();
  if (!ctx || !kernel || !count || !total_ms)
    return set_error(MOE_ERR_INVALID_ARG, "moe_ctx_kernel_time: NULL argument");
  int n = 0;
  double tot = 0.0;
  for (auto& r : ctx->recs) {
    if (std::strcmp(r.kernel, kernel) != 0) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return hip_error(e, "hipEventSynchronize");
    float ms = 0.0f;
    if ((e = hipEventElapsedTime(&ms, r.start, r.stop)) != hipSuccess) return hip_error(e, "hipEventElapsedTime");
    tot += ms;
    ++n;
  }
  *count = n;
  *total_ms = tot;
  return MOE_OK;
}

int moe_ctx_destroy(moe_ctx* ctx) {
  clear_error();
  if (!ctx) return MOE_OK;
  (void)hipDeviceSynchronize();
  for (auto& r : ctx->recs) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  for (auto e : ctx->spare_events) (void)hipEventDestroy(e);
  if (ctx->join_ev) (void)hipEventDestroy(ctx->join_ev);
  if (ctx->fork_ev) (void)hipEventDestroy(ctx->fork_ev);
  if (ctx->side) (void)hipStreamDestroy(ctx->side);
  if (ctx->d_err) (void)hipFree(ctx->d_err);
  delete ctx;
  return MOE_OK;
}

int moe_ctx_check(moe_ctx* ctx, void* stream) {
  clear_error();
  if (!ctx) return set_error(MOE_ERR_INVALID_ARG, "moe_ctx_check: ctx is NULL");
  int rc = ensure_device(ctx);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  int word = 0;
  hipError_t e = hipMemcpyAsync(&word, ctx->d_err, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_error(e, "moe_ctx_check");
  if (word != 0) {
    e = hipMemsetAsync(ctx->d_err, 0, sizeof(int), s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_error(e, "moe_ctx_check (clear)");
    if (word < 0)
      return set_error(MOE_ERR_INVALID_ARG, "an expert id outside [0, E) reached moe_permute; those pairs were left out");
    return set_error(MOE_ERR_NOT_RESIDENT,
                     "expert %d was routed to but has no VRAM slot (slot -1); its outputs are NaN",
                     word - 1);
  }
  return MOE_OK;
}

int moe_qtype_info(int qtype, int* block_elems, int* block_bytes) {
  clear_error();
  if (!qtype_supported(qtype))
    return set_error(MOE_ERR_UNSUPPORTED_QTYPE,
                     "block type %d is not supported (Q4_0=%d, Q4_1=%d, Q5_0=%d, Q5_1=%d, Q8_0=%d, Q4_K=%d, Q5_K=%d)",
                     qtype, MOE_QTYPE_Q4_0, MOE_QTYPE_Q4_1, MOE_QTYPE_Q5_0, MOE_QTYPE_Q5_1, MOE_QTYPE_Q8_0, MOE_QTYPE_Q4_K,
                     MOE_QTYPE_Q5_K);
  if (block_elems) *block_elems = qtype_is_k(qtype) ? kGroupWeights : kQK;
  if (block_bytes) *block_bytes = qtype_is_k(qtype) ? k_superblock_bytes(qtype) : ggml_block_bytes(qtype);
  return MOE_OK;
}

static int check_dims(const char* fn, int H, int I) {
  if (H <= 0 || I <= 0 || H % kGroupWeights || I % kGroupWeights)
    return set_error(MOE_ERR_INVALID_ARG, "%s: H=%d and I=%d must be positive multiples of %d",
                     fn, H, I, kGroupWeights);
  return MOE_OK;
}

int moe_slot_bytes(int qtype, int H, int I, size_t* out_bytes) {
  clear_error();
  if (!qtype_supported(qtype))
    return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "moe_slot_bytes: block type %d is not supported", qtype);
  int rc = check_dims("moe_slot_bytes", H, I);
  if (rc) return rc;
  if (!out_bytes) return set_error(MOE_ERR_INVALID_ARG, "moe_slot_bytes: out_bytes is NULL");
  *out_bytes = slot_bytes_of(qtype, H, I);
  return MOE_OK;
}

// ggml K-quant super-blocks [rows][cols/256] -> device groups: sub-block
// b's 32 codes (ggml: bytes 32 (b/2) + l of the nibbles, low nibble for even
// b, high for odd) as 16 bytes with element j in the low and element j + 16
// in the high nibble of byte j; Q5_K: then sub-block b's fifth bits (ggml:
// bit b of qh byte l) as a word with bit l for element l; then the 12 scale
// bytes, d and dmin unchanged.
static void pack_matrix_k(int qtype, int rows, int cols, const uint8_t* src, uint8_t* dst) {
  const int groups = cols / kGroupWeights;
  const int sbb = k_superblock_bytes(qtype);
  const bool has_qh = qtype_has_qh(qtype);
  const int qs_in = 16 + (has_qh ? 32 : 0);  // ggml: d, dmin, scales, [qh,] qs
  for (int r = 0; r < rows; ++r) {
    for (int g = 0; g < groups; ++g) {
      const uint8_t* sb = src + ((size_t)r * groups + g) * sbb;
      uint8_t* d = dst + (size_t)r * row_bytes(qtype, cols) + (size_t)g * group_bytes(qtype);
      const uint8_t* qs = sb + qs_in;
      for (int b = 0; b < kGroupBlocks; ++b) {
        uint8_t code[32];
        for (int l = 0; l < 32; ++l) {
          const uint8_t v = qs[32 * (b / 2) + l];
          code[l] = (b & 1) ? (v >> 4) : (v & 0x0F);
        }
        for (int j = 0; j < 16; ++j) d[16 * b + j] = (uint8_t)(code[j] | (code[j + 16] << 4));
        if (has_qh) {
          uint32_t word = 0;
          for (int l = 0; l < 32; ++l) word |= (uint32_t)((sb[16 + l] >> b) & 1) << l;
          std::memcpy(d + group_qh_off(qtype) + 4 * b, &word, 4);
        }
      }
      std::memcpy(d + group_ksc_off(qtype), sb + 4, 12);
      std::memcpy(d + group_d_off(qtype), sb, 2);
      std::memcpy(d + group_m_off(qtype), sb + 2, 2);
    }
  }
}

// ggml blocks [rows][cols/32] -> device layout (groups of 8 blocks: quant
// bytes, fifth-bit words, scales d, offsets m).
static void pack_matrix(int qtype, int rows, int cols, const uint8_t* src, uint8_t* dst) {
  if (qtype_is_k(qtype)) return pack_matrix_k(qtype, rows, cols, src, dst);
  const int qb = quant_bytes_per_block(qtype);
  const int bb = ggml_block_bytes(qtype);
  const bool has_m = qtype_has_min(qtype), has_qh = qtype_has_qh(qtype);
  const int qh_in = 2 + (has_m ? 2 : 0), qs_in = qh_in + (has_qh ? 4 : 0);  // field offsets in a ggml block
  const int groups = cols / kGroupWeights;
  const size_t gbytes = group_bytes(qtype);
  for (int r = 0; r < rows; ++r) {
    for (int g = 0; g < groups; ++g) {
      const uint8_t* s = src + ((size_t)r * (cols / kQK) + (size_t)g * kGroupBlocks) * bb;
      uint8_t* d = dst + (size_t)r * row_bytes(qtype, cols) + (size_t)g * gbytes;
      for (int b = 0; b < kGroupBlocks; ++b) {
        const uint8_t* blk = s + (size_t)b * bb;
        std::memcpy(d + (size_t)b * qb, blk + qs_in, qb);
        if (has_qh) std::memcpy(d + group_qh_off(qtype) + 4 * b, blk + qh_in, 4);
        std::memcpy(d + group_d_off(qtype) + 2 * b, blk, 2);
        if (has_m) std::memcpy(d + group_m_off(qtype) + 2 * b, blk + 2, 2);
      }
    }
  }
}

int moe_pack_matrix(int qtype, int rows, int cols, const void* blocks, void* dst, size_t dst_bytes) {
  clear_error();
  if (!qtype_supported(qtype))
    return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "moe_pack_matrix: block type %d is not supported", qtype);
  if (rows <= 0 || cols <= 0 || cols % kGroupWeights)
    return set_error(MOE_ERR_INVALID_ARG, "moe_pack_matrix: rows=%d, cols=%d (cols must be a multiple of %d)",
                     rows, cols, kGroupWeights);
  if (!blocks || !dst) return set_error(MOE_ERR_INVALID_ARG, "moe_pack_matrix: NULL buffer");
  if (dst_bytes < matrix_bytes(qtype, rows, cols))
    return set_error(MOE_ERR_WORKSPACE, "moe_pack_matrix: dst holds %zu bytes, needs %zu", dst_bytes,
                     matrix_bytes(qtype, rows, cols));
  pack_matrix(qtype, rows, cols, (const uint8_t*)blocks, (uint8_t*)dst);
  return MOE_OK;
}

int moe_pack_expert(int qtype, int H, int I, const void* gate_blocks, const void* up_blocks,
                    const void* down_blocks, void* dst, size_t dst_bytes) {
  clear_error();
  if (!qtype_supported(qtype))
    return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "moe_pack_expert: block type %d is not supported", qtype);
  int rc = check_dims("moe_pack_expert", H, I);
  if (rc) return rc;
  if (!gate_blocks || !up_blocks || !down_blocks || !dst)
    return set_error(MOE_ERR_INVALID_ARG, "moe_pack_expert: NULL buffer");
  if (dst_bytes < slot_bytes_of(qtype, H, I))
    return set_error(MOE_ERR_WORKSPACE, "moe_pack_expert: dst holds %zu bytes, one slot needs %zu",
                     dst_bytes, slot_bytes_of(qtype, H, I));
  uint8_t* d = (uint8_t*)dst;
  pack_matrix(qtype, I, H, (const uint8_t*)gate_blocks, d + slot_gate_off(qtype, H, I));
  pack_matrix(qtype, I, H, (const uint8_t*)up_blocks, d + slot_up_off(qtype, H, I));
  pack_matrix(qtype, H, I, (const uint8_t*)down_blocks, d + slot_down_off(qtype, H, I));
  return MOE_OK;
}

int moe_check_bank_types(int L, int n_per_layer, const int* qtypes, int* out_qtype) {
  clear_error();
  if (L < 1 || n_per_layer < 1 || !qtypes)
    return set_error(MOE_ERR_INVALID_ARG, "moe_check_bank_types: L=%d n_per_layer=%d", L, n_per_layer);
  const int q0 = qtypes[0];
  std::string bad;
  int n_bad = 0;
  for (int l = 0; l < L; ++l) {
    bool differs = false;
    for (int j = 0; j < n_per_layer; ++j) differs |= qtypes[l * n_per_layer + j] != q0;
    if (differs) {
      if (n_bad < 32) bad += (bad.empty() ? "" : ", ") + std::to_string(l);
      ++n_bad;
    }
  }
  if (n_bad)
    return set_error(MOE_ERR_MIXED_QTYPE,
                     "expert banks mix block types: layer(s) %s%s differ from layer 0's type %d; one slot pool "
                     "needs one type",
                     bad.c_str(), n_bad > 32 ? ", ..." : "", q0);
  if (!qtype_supported(q0))
    return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "moe_check_bank_types: block type %d is not supported", q0);
  if (out_qtype) *out_qtype = q0;
  return MOE_OK;
}

}  // extern "C"
