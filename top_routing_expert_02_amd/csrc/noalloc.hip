// The layer forward for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): moe_layer_forward with its workspace in a fixed device array
// of this library instead of a caller's buffer.
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds one copy of MOE_NOALLOC_SCRATCH_BYTES from the moment the
// code object is loaded there until the process ends. Host code must not
// use the array's name as a device address: the first call on a device
// looks up that device's copy with hipGetSymbolAddress (with the device
// current) and keeps the address; kernels only ever receive that address.
//
// Every call on one GPU shares its array, and each call leaves its contents
// behind. Nothing in it has to start at zero: every layer kernel writes
// what it later reads (the per-tile histograms that the top-k adds into are
// cleared by the logits kernel of the same call). Calls that overlap on one
// GPU (two streams, two host threads) race on the array.
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace {

__device__ __attribute__((aligned(256))) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {nullptr};
std::mutex g_scratch_mutex;

// this device's copy of the array (looked up once per device), or null
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int32_t moe_layer_forward_noalloc(const moe_config* cfg, const void* x, const void* W_r,
                                             const float* b_r, const void* W1, const float* b1,
                                             const void* W2, const float* b2, void* y,
                                             const moe_route_info* info, hipStream_t stream) {
  // sizes first: a layer whose workspace exceeds the array is refused before
  // any device call
  size_t need = 0;
  const int32_t st = moe_workspace_size(cfg, &need);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (need > static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES)) return MOE_ERR_WORKSPACE;
  hipError_t err = hipSuccess;
  void* ws = scratch_on_current_device(&err);
  if (ws == nullptr) return MOE_ERR_HIP;
  return moe_layer_forward(cfg, x, W_r, b_r, W1, b1, W2, b2, y, info, ws,
                           static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES), nullptr, nullptr, stream);
}
