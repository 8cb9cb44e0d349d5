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
bool linear_mfma_supported(const LinearArgs& a);
int launch_linear_mfma(const LinearArgs& a, hipStream_t s);
bool linear_pp_supported(const LinearArgs& a);
int launch_linear_pp(const LinearArgs& a, hipStream_t s);

}  // namespace dstar
