// moe_decode_layer_static: the decode layer of moe_decode_layer with its
// workspace in a library-owned static device array instead of a buffer the
// caller allocates, for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).
//
// The array lives at file scope, so every GPU the library runs on holds its
// own copy, at its own address, until the process ends.  In host code the
// array's name is only a host-side stand-in: its device address is looked
// up once per device with hipGetSymbolAddress (from moe_ctx_create, with the
// device current) and only that address is handed to kernels.
#include <mutex>

#include "ffn.h"

namespace moe {
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;
}  // namespace moe

// decode h rows (T*k x I fp32) of the layer in flight on this device
static __device__ __align__(256) uint8_t scratch[moe::kStaticScratchBytes];

namespace moe {

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of this device's `scratch`, resolved on the first call for
// the device (the caller has made `device` current).
int static_scratch_init(int device, void** out) {
  if (device < 0 || device >= kMaxDevices)
    return set_error(MOE_ERR_INVALID_ARG, "static scratch: device %d beyond %d", device, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_error(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return set_error(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_static_scratch_bytes(void) { return kStaticScratchBytes; }

extern "C" int moe_decode_layer_static(moe_ctx* ctx, const moe_ffn_args* args, const float* router_w,
                                       const float* bias, const float* logits_in, float* logits_out,
                                       int32_t* topk_ids, int32_t* pair_pos, void* stream) {
  clear_error();
  if (!ctx || !args) return set_error(MOE_ERR_INVALID_ARG, "moe_decode_layer_static: ctx or args is NULL");
  if (!ctx->d_scratch)
    return set_error(MOE_ERR_HIP, "moe_decode_layer_static: the context has no static scratch address");
  moe_ffn_args a = *args;
  a.ws = ctx->d_scratch;
  a.ws_bytes = kStaticScratchBytes;
  size_t need = 0;
  int rc = moe_expert_ffn_workspace_size(&a, &need);
  if (rc) return rc;
  if (need > kStaticScratchBytes)
    return set_error(MOE_ERR_WORKSPACE,
                     "moe_decode_layer_static: T=%d k=%d I=%d needs %zu bytes of scratch; the static scratch "
                     "holds %zu (T*k*I*4 bytes must fit)",
                     a.T, a.k, a.I, need, kStaticScratchBytes);
  return moe_decode_layer(ctx, &a, router_w, bias, logits_in, logits_out, topk_ids, pair_pos, stream);
}
