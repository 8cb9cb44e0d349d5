// Elementwise GELU (the activation between the two linears of a DiT MLP,
// which DSTAR fuses into the first linear through its vector unit: §4.2
// "Design of VPU", §4.3 "Linear Operation").  The fused form is the epilogue
// of stage 3 (gelu_out); this stand-alone kernel makes the GELU of a cached
// output, e.g. the previous step's input of the second linear when a chain
// of timesteps starts.  Same function as gelu_of: float64 evaluation, one
// rounding to float32.
#include "fmdq_internal.h"

namespace dstar {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void gelu_kernel(const float* y, float* g, int64_t n) {
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4*>(y) + i);
    f4 o;
    o.x = gelu_of(v.x);
    o.y = gelu_of(v.y);
    o.z = gelu_of(v.z);
    o.w = gelu_of(v.w);
    __builtin_nontemporal_store(o, reinterpret_cast<f4*>(g) + i);
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 4 * n4) g[4 * n4 + threadIdx.x] = gelu_of(y[4 * n4 + threadIdx.x]);
}

}  // namespace

int launch_gelu(const float* y, float* g, int64_t n, hipStream_t s) {
  if (n == 0) return DSTAR_OK;
  const int64_t blocks = (n / 4 + 255) / 256;
  const int64_t grid = blocks < 1 ? 1 : (blocks > 8192 ? 8192 : blocks);
  hipLaunchKernelGGL(gelu_kernel, dim3((unsigned)grid), dim3(256), 0, s, y, g, n);
  return check_launch("fmdq_gelu");
}

}  // namespace dstar
