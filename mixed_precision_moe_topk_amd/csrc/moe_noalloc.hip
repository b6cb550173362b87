// The run call for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation):
// moe_run_noalloc runs the same kernels as moe_run_ws with a workspace that
// lives in a file-scope device array of fixed size, so the call itself
// allocates nothing.
//
// Each device the library runs on holds its own copy of `scratch` for the
// life of the process.  The array's name in host code is only a host-side
// stand-in, not a device address: the device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/moe.h"
#include "moe_common.h"

namespace moe {
moe_status run_ws_untraced(const moe_dims* dims, const void* hidden, int64_t num_tokens,
                           const float* router_logits, const void* weights, const void* scales,
                           int32_t top_k, void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);
moe_status set_error(moe_status st, const char* msg);
}  // namespace moe

namespace {

constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of this device's `scratch` (looked up on the first call on
// the device, with that device current).
moe_status scratch_of_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return moe::set_error(MOE_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return moe::set_error(MOE_ERR_UNSUPPORTED, "device index beyond the static scratch table");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return moe::set_error(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) failed");
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_run_noalloc(const moe_dims* dims, const void* hidden,
                                      int64_t num_tokens, const float* router_logits,
                                      const void* weights, const void* scales, int32_t top_k,
                                      void* out, hipStream_t stream) {
  size_t need = 0;
  moe_status st = moe_workspace_query(dims, num_tokens, top_k, &need);
  if (st != MOE_OK) return st;
  if (need > kScratchBytes) {
    char msg[192];
    snprintf(msg, sizeof(msg),
             "moe_run_noalloc: the layer needs a %zu-byte workspace, the static scratch holds "
             "%zu bytes (use moe_run_ws with a caller workspace)",
             need, kScratchBytes);
    return moe::set_error(MOE_ERR_WORKSPACE, msg);
  }
  if (num_tokens == 0) return moe_run_ws(dims, hidden, 0, router_logits, weights, scales, top_k,
                                         out, nullptr, 0, stream);
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != MOE_OK) return st;
  // the workspace needs no initialisation: every region is written before
  // it is read within the call
  return moe::run_ws_untraced(dims, hidden, num_tokens, router_logits, weights, scales, top_k,
                              out, ws, kScratchBytes, stream);
}
