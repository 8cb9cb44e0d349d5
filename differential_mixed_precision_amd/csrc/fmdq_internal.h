// Internal declarations shared by the HIP sources of the FMDQ library.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <cstdarg>
#include "dstar_fmdq.h"

namespace dstar {

// Records a thread-local error message and returns `code`.
int set_error(int code, const char* fmt, ...);
void clear_error();

// Checks hipGetLastError() after a launch; returns DSTAR_OK or DSTAR_EHIP.
int check_launch(const char* what);

__host__ __device__ inline int64_t n_tiles(int64_t rows, int64_t T) { return (rows + T - 1) / T; }

// Validated launch descriptions (sizes already checked by the API layer).
struct QuantizeArgs {
  const float* x_t;
  const float* x_prev;
  int8_t* codes;
  uint8_t* tags;
  int8_t* acodes;
  int8_t* hcodes;     // digit planes [2][n_t][K][T] (with acodes)
  int64_t plane;      // n_t * K * T: offset of the second plane
  uint32_t* bit_hist;
  int64_t rows;
  int32_t K;
  int32_t T;
  float base;
  float inv_base;
  const float* base_dev;   // non-NULL: base read from device memory (dynamic base)
  int32_t k0;
};
int launch_quantize(const QuantizeArgs& a, hipStream_t s);

struct BucketArgs {
  const uint8_t* tags;
  uint16_t* perm;
  int32_t* group_off;
  int64_t n_tiles;
  int32_t K;
};
int launch_bucket(const BucketArgs& a, hipStream_t s);
struct SliceArgs {
  const int8_t* codes;
  const uint8_t* tags;
  uint32_t* entries;
  uint8_t* slices;
  int32_t* slice_off;
  int64_t n_tiles;
  int32_t K;
  int32_t T;
};
int launch_slices(const SliceArgs& a, hipStream_t s);

struct LinearArgs {
  const int8_t* codes;
  const uint16_t* perm;
  const int32_t* group_off;
  const int8_t* acodes;
  const int8_t* hcodes;
  const int8_t* w;
  const int8_t* w_t;
  const float* w_scale;
  const float* y_prev;
  float* y_out;
  int32_t* acc_dbg;        // per-group accumulator dump (general kernel only)
  int64_t* s_dbg;          // exact S dump, written by whichever kernel runs
  int32_t dbg_lo;
  int32_t dbg_hi;
  int64_t rows;
  int32_t K;
  int32_t N;
  int32_t T;
  double base;
  const float* base_dev;   // non-NULL: base read from device memory (dynamic base)
  float* gelu_out;         // non-NULL: GELU(Y_t) is stored here as well
};
int launch_linear(const LinearArgs& a, hipStream_t s);
// The exact S of rows t0 .. t0 + TR − 1 of token tile tau at column n, for a
// tile the product kernels cannot prove exact in int32: every channel's
// shift-aligned value a = q·2^e = d0 + 2^7·d1 + 2^15·d2 is rebuilt from the
// aligned codes (d0) and the digit planes, whose entries exist only for the
// sub-channels with PoT ≥ 7 (d1) and PoT ≥ 14 (d2), and S = Σ_k a·W[k][n]
// is summed in int64 (|a| ≤ 2^21, |W| ≤ 128, K < 2^16).  The channels are
// walked bin by bin in perm order: bin b holds FPoT tag g = b / 4 and
// precision code pc = 3 − b mod 4, so PoT = (15 − g) + 2·pc.  This is
// Σ_g 2^(15−g) · Σ_{k in group g} q·W of §3.1 step 5 regrouped by channel.
template <int T, int TR>
__device__ __forceinline__ void aligned_tile_sums(const LinearArgs& a, const int32_t* off, int64_t tau, int t0,
                                                  int64_t n, int64_t (&sum)[TR]) {
  const int64_t K = a.K, N = a.N;
  const uint16_t* pm = a.perm + tau * K;
  const int8_t* ac = a.acodes + (tau * T + t0) * K;           // row t0 of the tile, [rows][K]
  const int8_t* h1 = a.hcodes + tau * K * T + t0;             // [n_t][K][T] planes
  const int8_t* h2 = h1 + n_tiles(a.rows, T) * K * T;
#pragma unroll
  for (int t = 0; t < TR; ++t) sum[t] = 0;
  for (int b = 0; b < DSTAR_FMDQ_NUM_BINS; ++b) {
    const int lo = off[b], hi = off[b + 1];
    if (lo == hi) continue;
    const int pot = (DSTAR_FMDQ_TAG_OFFSET - (b >> 2)) + 2 * (3 - (b & 3));
    for (int j = lo; j < hi; ++j) {
      const int64_t k = pm[j];
      const int64_t wv = (int64_t)a.w[k * N + n];
      int32_t av[TR];
#pragma unroll
      for (int t = 0; t < TR; ++t) av[t] = (int32_t)ac[t * K + k];
      if (pot >= 7) {
#pragma unroll
        for (int v = 0; v < TR / 16; ++v) {
          const int4 c = reinterpret_cast<const int4*>(h1 + k * T)[v];
          const int words[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
          for (int q = 0; q < 16; ++q) av[16 * v + q] += 128 * (int32_t)(int8_t)(words[q >> 2] >> (8 * (q & 3)));
        }
      }
      if (pot >= 14) {
#pragma unroll
        for (int v = 0; v < TR / 16; ++v) {
          const int4 c = reinterpret_cast<const int4*>(h2 + k * T)[v];
          const int words[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
          for (int q = 0; q < 16; ++q) av[16 * v + q] += 32768 * (int32_t)(int8_t)(words[q >> 2] >> (8 * (q & 3)));
        }
      }
#pragma unroll
      for (int t = 0; t < TR; ++t) sum[t] += (int64_t)av[t] * wv;
    }
  }
}
struct BaseArgs {
  const float* x_t;
  const float* x_prev;
  uint32_t* base_bits;     // the float32 result, handled as its bit pattern
  int64_t rows;
  int32_t K;
  int32_t T;
  float fallback;
};
int launch_dynamic_base(const BaseArgs& a, hipStream_t s);
// GELU in its tanh form, y / (1 + exp(-2u)) with u = c·(y + a·y³), evaluated
// in float64 (the cube as (y·y)·y) and rounded once to float32: the activation
// between the two linears of the MLP, fused into the first one's epilogue.
__device__ __forceinline__ float gelu_of(float yf) {
  const double y = (double)yf;
  const double u = __dmul_rn(0.7978845608028654,
                             __dadd_rn(y, __dmul_rn(0.044715, __dmul_rn(__dmul_rn(y, y), y))));
  return (float)__ddiv_rn(y, __dadd_rn(1.0, exp(__dmul_rn(-2.0, u))));
}
int launch_gelu(const float* y, float* g, int64_t n, hipStream_t s);
int launch_pack_weights(int32_t K, int32_t N, const int8_t* w, int8_t* w_t, hipStream_t s);
int launch_linear_general(const LinearArgs& a, hipStream_t s);

// Byte offsets of the intermediates in the workspace of the one-call layer
// (each 256-byte aligned): codes, aligned codes, digit planes, tags, bucket
// ids, bin offsets.
struct LayerWorkspace {
  int64_t codes, acodes, hcodes, tags, perm, off, total;
};
LayerWorkspace layer_workspace(int64_t nt, int64_t K, int64_t T);
// The three stages on the caller's stream with the intermediates in
// `workspace` (checked: non-NULL, 256-byte aligned, large enough).
int layer_impl(const dstar_fmdq_params* p, int32_t N, const float* x_t, const float* x_prev,
               const int8_t* w, const int8_t* w_t, const float* w_scale, const float* y_prev,
               float* y_out, uint32_t* bit_hist, void* workspace, int64_t workspace_bytes,
               void* stream);
int cu_count();   // compute units of the current device
bool linear_mfma_supported(const LinearArgs& a);
int launch_linear_mfma(const LinearArgs& a, hipStream_t s);
bool linear_pp_supported(const LinearArgs& a);
int launch_linear_pp(const LinearArgs& a, hipStream_t s);

}  // namespace dstar
