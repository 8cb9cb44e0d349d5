// Stage 3 dispatch: the MFMA kernel for token tiles of 32 or 64 rows, K a
// multiple of 64, with the aligned codes, digit planes and W^T given; the
// general kernel for other shapes and whenever the per-group accumulators are
// dumped (only the general kernel has them).  The S dump is written by
// whichever kernel runs.
#include "fmdq_internal.h"

namespace dstar {

int launch_linear(const LinearArgs& a, hipStream_t s) {
  if (a.acc_dbg == nullptr && linear_mfma_supported(a)) return launch_linear_mfma(a, s);
  return launch_linear_general(a, s);
}

}  // namespace dstar
