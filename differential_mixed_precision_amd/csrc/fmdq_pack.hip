// Weight preparation: w_t[n][k] = w[k][n].  The dense GEMM of stage 3 reads
// both of its operands with the reduction index innermost; the layer's
// weights are static, so this copy is made once per layer.
//
// 64 × 64-byte tiles through LDS: coalesced reads along n, coalesced writes
// along k.
#include "fmdq_internal.h"

namespace dstar {
namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void pack_weights_kernel(int32_t K, int32_t N, const int8_t* w,
                                                                int8_t* w_t) {
  __shared__ int8_t tile[kTile][kTile + 4];
  const int64_t k0 = (int64_t)blockIdx.y * kTile;
  const int64_t n0 = (int64_t)blockIdx.x * kTile;
  for (int idx = threadIdx.x; idx < kTile * kTile; idx += kThreads) {
    const int r = idx / kTile, c = idx % kTile;   // r: k, c: n
    const int64_t k = k0 + r, n = n0 + c;
    tile[r][c] = (k < K && n < N) ? w[k * N + n] : (int8_t)0;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kTile * kTile; idx += kThreads) {
    const int r = idx / kTile, c = idx % kTile;   // r: n, c: k
    const int64_t n = n0 + r, k = k0 + c;
    if (n < N && k < K) w_t[n * K + k] = tile[c][r];
  }
}

}  // namespace

int launch_pack_weights(int32_t K, int32_t N, const int8_t* w, int8_t* w_t, hipStream_t s) {
  const dim3 grid((unsigned)((N + kTile - 1) / kTile), (unsigned)((K + kTile - 1) / kTile));
  hipLaunchKernelGGL(pack_weights_kernel, grid, dim3(kThreads), 0, s, K, N, w, w_t);
  return check_launch("fmdq_pack_weights");
}

}  // namespace dstar
