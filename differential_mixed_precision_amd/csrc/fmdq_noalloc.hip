// The one-call layer without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc): the intermediates live in a file-scope
// device array of kScratchBytes that every call on a GPU shares.
//
// The array's name is a host-side stand-in in host code, not a device
// address: its address on a device comes from hipGetSymbolAddress, taken once
// per device (with that device current) on the first call there, kept in
// g_scratch[], and used for every kernel argument.  Nothing here allocates.
// Every call on one GPU uses the same array, so calls that overlap in time on
// one GPU race; the stages write every intermediate they read, so nothing has
// to be cleared between calls.
#include <mutex>

#include "fmdq_internal.h"

namespace dstar {
namespace {

constexpr int64_t kScratchBytes = DSTAR_FMDQ_NOALLOC_MAX_BYTES;   // 64 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up once).
int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(DSTAR_EHIP, "layer_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(DSTAR_EUNSUPPORTED, "layer_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return set_error(DSTAR_EHIP, "layer_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DSTAR_OK;
}

}  // namespace
}  // namespace dstar

using namespace dstar;

extern "C" int dstar_fmdq_layer_noalloc(const dstar_fmdq_params* p, int32_t N, const float* x_t,
                                        const float* x_prev, const int8_t* w, const int8_t* w_t,
                                        const float* w_scale, const float* y_prev, float* y_out,
                                        uint32_t* bit_hist, void* stream) {
  clear_error();
  const int64_t need = dstar_fmdq_layer_workspace_size(p);
  if (need < 0) return (int)need;
  if (need > kScratchBytes)
    return set_error(DSTAR_EINVAL, "layer_noalloc: these sizes need %lld bytes of scratch, above its %lld",
                     (long long)need, (long long)kScratchBytes);
  void* ws = nullptr;
  if (int rc = scratch_on_current_device(&ws)) return rc;
  return layer_impl(p, N, x_t, x_prev, w, w_t, w_scale, y_prev, y_out, bit_hist, ws, kScratchBytes, stream);
}
