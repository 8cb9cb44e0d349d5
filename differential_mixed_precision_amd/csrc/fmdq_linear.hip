// Stage 3 dispatch.
#include "fmdq_internal.h"

namespace dstar {

int launch_linear_general(const LinearArgs& a, hipStream_t s);

int launch_linear(const LinearArgs& a, hipStream_t s) { return launch_linear_general(a, s); }

}  // namespace dstar
