// moe_forward_windows_noalloc: moe_forward_windows for callers that cannot
// allocate device memory (code under stream capture, tight serving loops,
// harnesses that forbid allocation). Its workspace is a fixed array of
// device memory defined here, one copy per GPU, so the call allocates
// nothing: the caller passes only the layer, inputs and outputs.
//
// Host code never uses the array's name as a device address (on the host
// it is a stand-in symbol): the first call on each device, with that device
// current, asks the runtime for the array's address on that device
// (hipGetSymbolAddress) and keeps it; every later call on that device passes
// the kept address to the kernels, exactly where moe_forward_windows passes
// the caller's workspace.
//
// The array keeps the last call's contents. Nothing in it needs clearing
// between calls: it starts zero when the code object is loaded, the router's
// hand-off words are tagged with a call counter kept beside them, and the
// fp16 h buffers are written before they are read in every call. Calls that
// overlap on one GPU (on two streams, or from two threads) share the array
// and race.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "moe_host.h"

namespace {

// Stated maximum: the 16-row decode workspace of the layers this call
// serves. The qwen3_5-MoE 35B-A3B shapes (hidden 2048, 256 experts, top-8,
// intermediate 512) need 329,216 bytes; larger layers are refused.
constexpr uint64_t kScratchBytes = 512u << 10;
constexpr int kMaxDevices = 64;
constexpr int kWindowRows = 16;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (null until resolved)

// The array's address on the current device, resolved once per device.
int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    moe::set_error(std::string("moe_forward_windows_noalloc: hipGetDevice: ") + hipGetErrorName(e));
    return MOE_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    moe::set_error("moe_forward_windows_noalloc: device index " + std::to_string(dev) + " outside 0.." +
                   std::to_string(kMaxDevices - 1));
    return MOE_EINVAL;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      moe::set_error(std::string("moe_forward_windows_noalloc: hipGetSymbolAddress: ") + hipGetErrorName(e));
      return MOE_EHIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_windows_noalloc(const moe_layer* layer, const void* x, int rows,
                                           const float* logit_bias, int32_t* ids, float* p,
                                           float* shared_gate, float* y, void* stream) {
  if (!layer) {
    moe::set_error("moe_forward_windows_noalloc: layer is NULL");
    return MOE_EINVAL;
  }
  int st = moe::validate_desc(&layer->d);
  if (st) return st;
  if (rows < 1 || rows > 65536) {
    moe::set_error("moe_forward_windows_noalloc: rows outside 1..65536");
    return MOE_EINVAL;
  }
  const uint64_t need = moe::decode_ws_layout(&layer->d, std::min(rows, kWindowRows)).total;
  if (need > kScratchBytes) {
    moe::set_error("moe_forward_windows_noalloc: this layer's windows need " + std::to_string(need) +
                   " bytes of workspace, above the fixed " + std::to_string(kScratchBytes) +
                   "-byte device array; use moe_forward_windows with a workspace");
    return MOE_ENOSPACE;
  }
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st) return st;
  // an earlier call's router failure is not carried into this call (its
  // callers cannot clear the count); failed rows show as ids -1 and NaN
  return moe::forward_windows_impl(layer, x, rows, logit_bias, ids, p, shared_gate, y, ws, kScratchBytes,
                                   stream, 0);
}
