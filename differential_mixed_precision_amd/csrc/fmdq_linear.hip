// Stage 3 dispatch.  Two MFMA kernels compute the same exact integer sum:
//   - the ping-pong kernel (256 × 256 output blocks, one workgroup of eight
//     waves per CU, the two waves of each SIMD alternating matrix and memory
//     phases): the faster dense loop, but its Y_{t-1}/Y_t stream cannot
//     overlap another workgroup's matrix work on the same CU;
//   - the two-workgroups-per-CU kernel (128 × 256 blocks of four waves, or
//     128 × 128 where the wider blocks would number fewer than the CUs),
//     whose workgroups hide each other's Y stream.
// Measured on MI355X over the five workloads: the ping-pong kernel is faster
// where the reduction is long (K ≥ 4096, so the matrix work dominates the Y
// stream) and its blocks fill at least half of the CUs; the other kernel
// everywhere else.  They need T of 32 (the ping-pong one) or 16/32/64, K a
// multiple of 16, the aligned codes, digit planes and W^T, and buffers small
// enough for 32-bit offsets.  The general
// kernel runs for other shapes and whenever the per-group accumulators are
// dumped (only it keeps one accumulator per FPoT group); it alone reads the
// plain codes, which the MFMA kernels do not need.  The S dump is written by
// whichever kernel runs.
#include <atomic>

#include "fmdq_internal.h"

namespace dstar {

// Compute units of the current device (looked up once per device; threads
// that race on the first lookup store the same value).
int cu_count() {
  static std::atomic<int> counts[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = counts[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    counts[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int launch_linear(const LinearArgs& a, hipStream_t s) {
  if (a.acc_dbg == nullptr && linear_pp_supported(a) && a.T == 32 && a.K >= 4096) {
    const int64_t blocks = ((n_tiles(a.rows, a.T) + 7) / 8) * ((a.N + 255) / 256);
    if (2 * blocks >= cu_count()) return launch_linear_pp(a, s);
  }
  if (a.acc_dbg == nullptr && linear_mfma_supported(a)) return launch_linear_mfma(a, s);
  if (a.codes == nullptr)
    return set_error(DSTAR_ENULL,
                     "fmdq_linear: codes are needed here (the per-group kernel runs: acc_dbg given, no W^T, "
                     "or a shape the MFMA kernels do not take)");
  return launch_linear_general(a, s);
}

}  // namespace dstar
