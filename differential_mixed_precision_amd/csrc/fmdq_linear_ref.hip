// Stage 3 of the FMDQ differential linear, general kernel: grouped integer GEMM
// with shift alignment and the fused dequantize / reverse-differential
// epilogue (DSTAR, arXiv 2607.15846: §3.1 step 5 and Fig. 6; §4.2 MPU with its
// inverse quantization and accumulation units; §4.3 reverse differential fused
// into the GEMM).
//
// This kernel handles every case the ABI allows (any number of FPoT groups per
// tile, any T, any N) and writes the optional accumulator dump.  A thread owns
// one output column of one token tile and walks the tile's channels in bucket
// order, one group after the other: the group sum is kept in int32, and at the
// end of a group it is shifted into the int64 sum S (the left shift by the
// FPoT difference of DSTAR §3.1 step 5, written relative to tag 15).
#include "fmdq_internal.h"

namespace dstar {
namespace {

constexpr int kThreads = 256;

template <int T>
__global__ __launch_bounds__(kThreads) void linear_general_kernel(LinearArgs a, int64_t n_work,
                                                                  int32_t col_blocks) {
  const int64_t K = a.K, N = a.N;
  for (int64_t wi = blockIdx.x; wi < n_work; wi += gridDim.x) {
    const int64_t tile = wi / col_blocks;
    const int64_t n = (wi - tile * col_blocks) * kThreads + threadIdx.x;
    const bool valid = n < N;
    const int32_t* off = a.group_off + tile * (DSTAR_FMDQ_NUM_BINS + 1);
    const uint16_t* pm = a.perm + tile * K;
    const int8_t* cd = a.codes + tile * K * T;
    const int64_t r0 = tile * T;
    const int nrows = (int)((a.rows - r0) < T ? (a.rows - r0) : T);
    const bool dump = a.acc_dbg != nullptr && tile >= a.dbg_lo && tile < a.dbg_hi;
    int64_t s[T];
#pragma unroll
    for (int t = 0; t < T; ++t) s[t] = 0;
    for (int g = 0; g < DSTAR_FMDQ_NUM_TAGS; ++g) {
      const int lo = off[4 * g], hi = off[4 * g + 4];
      if (lo == hi && !dump) continue;
      int32_t acc[T];
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t] = 0;
      for (int j = lo; j < hi; ++j) {
        const int64_t k = pm[j];
        const int32_t wv = valid ? (int32_t)a.w[k * N + n] : 0;
        const int4* c4 = reinterpret_cast<const int4*>(cd + k * T);
#pragma unroll
        for (int v = 0; v < T / 16; ++v) {
          const int4 c = c4[v];
          const int words[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
          for (int b = 0; b < 16; ++b) {
            const int32_t q = (int32_t)(int8_t)(words[b >> 2] >> (8 * (b & 3)));
            acc[16 * v + b] += q * wv;
          }
        }
      }
#pragma unroll
      for (int t = 0; t < T; ++t) s[t] += (int64_t)acc[t] << (DSTAR_FMDQ_TAG_OFFSET - g);
      if (dump && valid) {
        int32_t* dst = a.acc_dbg + ((tile - a.dbg_lo) * DSTAR_FMDQ_NUM_TAGS + g) * (int64_t)T * N + n;
#pragma unroll
        for (int t = 0; t < T; ++t) dst[t * N] = acc[t];
      }
    }
    if (!valid) continue;
    if (a.s_dbg != nullptr && tile >= a.dbg_lo && tile < a.dbg_hi) {
      int64_t* dst = a.s_dbg + (tile - a.dbg_lo) * (int64_t)T * N + n;
#pragma unroll
      for (int t = 0; t < T; ++t) dst[t * N] = s[t];
    }
    const double base = a.base_dev != nullptr ? (double)*a.base_dev : a.base;
    const double ws = (double)a.w_scale[n];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (t < nrows) {
        const int64_t idx = (r0 + t) * N + n;
        const double d = __dmul_rn(__dmul_rn((double)s[t], base), ws);
        const float y = (float)__dadd_rn((double)a.y_prev[idx], d);
        a.y_out[idx] = y;
        if (a.gelu_out != nullptr) a.gelu_out[idx] = gelu_of(y);
      }
    }
  }
}

template <int T>
int launch_t(const LinearArgs& a, hipStream_t s) {
  const int64_t nt = n_tiles(a.rows, T);
  const int32_t col_blocks = (a.N + kThreads - 1) / kThreads;
  const int64_t n_work = nt * col_blocks;
  const int64_t grid = n_work < 8192 ? n_work : 8192;
  hipLaunchKernelGGL(linear_general_kernel<T>, dim3((unsigned)grid), dim3(kThreads), 0, s, a,
                     n_work, col_blocks);
  return check_launch("fmdq_linear (general)");
}

}  // namespace

int launch_linear_general(const LinearArgs& a, hipStream_t s) {
  switch (a.T) {
    case 16: return launch_t<16>(a, s);
    case 32: return launch_t<32>(a, s);
    case 64: return launch_t<64>(a, s);
    default: return set_error(DSTAR_EUNSUPPORTED, "token_tile %d not supported", a.T);
  }
}

}  // namespace dstar
