// Sparse Attention Reuse with FMDQ-INT8 operands (DSTAR, arXiv 2607.15846:
// §3.2 "Sparse Attention Reuse", Fig. 8; §4.3 "Attention Operation", Fig. 13).
//
// Kernels:
//   qquant  FMDQ-INT8 of Q: one wave per 32-row token tile, a lane per channel
//           (two channel passes), the tile's rows streamed with coalesced loads.
//   kquant  int8 of K with a scale per key: eight lanes per key row (one wave
//           per 8 rows when d is not a multiple of 4 or K is not 16-byte
//           aligned).
//   vquant  int8 of V with a scale per channel: a column-maximum pass (partial
//           maxima of 256-row chunks lowered into the scale buffer by atomic
//           max on the float bits), a quantize pass that writes the codes
//           channel-major, and a pass that turns the maxima into scales.
//   scores  cached step: one wave per (image·head, 32-row token tile); three
//           sweeps over the kept key blocks of its query block (row maximum of
//           the logits, sum of the fixed-point exponentials, then P and its
//           FMDQ-INT8 codes), each recomputing the exact integer scores; the
//           next block's K fragments are loaded while one is computed.  Waves
//           take the query blocks with the most kept key blocks first.
//   pv      cached and reused steps: one wave per (image·head, token tile),
//           one int32 MFMA accumulator per (column tile, digit plane) over all
//           kept keys, combined in int64 at the end.
// Both run two waves per SIMD: the number of digit planes a wave needs is
// found first and selects a templated body, so the common cases (two planes
// of a_Q, three of a_P) keep few registers.
//
// Exact integer products on int8 MFMAs.  An FMDQ operand value in integer
// units is a = code·2^PoT (|code| ≤ 64, PoT ≤ 21, so |a| ≤ 2^27).  It is split
// into signed base-256 digits a = Σ_j 2^(8j)·d_j (d_j in [-128, 127]); each
// digit plane is an int8 matrix, and one v_mfma_i32_32x32x32_i8 chain per
// plane gives an exact int32 partial product (|Σ| ≤ 128·127·128 < 2^22 per
// block of keys).  scores combines two planes in int32 (|S| < 2^30) and more
// in int64; pv keeps one int32 accumulator per plane over all kept keys
// (|Σ| ≤ 128·127·2^16 < 2^31) and combines them in int64 once.  The planes a
// tile needs follow from its
// largest PoT (one for PoT 0, two up to 8, three up to 16, four beyond), so
// typical Q tiles take two and P tiles two or three.  The MFMA operands are
// loaded straight from global memory in the fragment layout (16 consecutive
// int8 per lane: A row = lane % 32, B column = lane % 32, k = 16·(lane / 32)):
// rows of qcodes/kcodes and of the P cache blocks and channel rows of the
// transposed V codes are contiguous along k.
#include <cmath>
#include <initializer_list>
#include <utility>

#include "dstar_sar.h"
#include "fmdq_internal.h"

namespace dstar {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBlock = DSTAR_SAR_BLOCK;
constexpr int kTile = DSTAR_SAR_TILE;
constexpr int kPlanes = 4;                     // digit planes of |a| ≤ 2^27
constexpr int kP8 = 6;                         // log2 of the 8-bit ceiling 64
constexpr int kPotMax = DSTAR_FMDQ_POT_MAX;    // 21
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// exp32 constants, float32 (hex literals so that both implementations start
// from the same bits): log2(e); ln 2 = LN2_HI + LN2_LO with LN2_HI = 355/512,
// whose product with a small integer n is exact; Taylor coefficients of e^r
// from 1/7! down to 1, here times 2^36 (the fixed-point scale of E): a
// power-of-two factor on every coefficient scales every Horner step by it
// exactly, so p·2^36 comes out of the polynomial with the same bits.
constexpr float kLog2e = 0x1.715476p+0f;
constexpr float kLn2Hi = 0x1.63p-1f;
constexpr float kLn2Lo = -0x1.bd0106p-13f;
constexpr float kExpScale = (float)(1ull << DSTAR_SAR_EXP_FRAC);
static_assert(DSTAR_SAR_EXP_FRAC == 36, "coefficient scale");
constexpr float kXMin = -26.0f;       // exp32 cut-off: E = 0 below it
constexpr float kXSafe = 16384.0f;    // |x| below which no clamp is needed

// E = rint(exp32(x)·2^36) as a float (an exact integer ≤ 2^36), x ≤ 0.
// exp32: Cody–Waite reduction n = rint(x·log2 e), r = (x − n·LN2_HI) −
// n·LN2_LO, then the degree-7 Taylor polynomial of e^r by Horner's rule, one
// fused multiply-add per step, each rounded once to float32; e = p·2^n.
// x − n·LN2_HI is one fused multiply-add: while |n| < 2^15 the product
// n·LN2_HI is exact, so it rounds the same value as a product followed by
// a difference.  The cut-off needs no clamp for −kXSafe ≤ x < −26: there
// n ≤ −38, p·2^(n+36) ≤ 1.42/4 and rint gives 0, as below the cut-off.
// Farther out the reduction loses the leading bits of x and the polynomial
// can overflow, so kClamp raises x to −26 first (E(−26) = 0).
template <bool kClamp>
__device__ __forceinline__ float exp_fixed(float x) {
  if constexpr (kClamp) x = fmaxf(x, kXMin);
  const float n = rintf(__fmul_rn(x, kLog2e));
  float r = __builtin_fmaf(-n, kLn2Hi, x);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float p = 0x1.a01a02p-13f * kExpScale;                 // 1/5040
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f * kExpScale);  // 1/720
  p = __builtin_fmaf(p, r, 0x1.111112p-7f * kExpScale);   // 1/120
  p = __builtin_fmaf(p, r, 0x1.555556p-5f * kExpScale);   // 1/24
  p = __builtin_fmaf(p, r, 0x1.555556p-3f * kExpScale);   // 1/6
  p = __builtin_fmaf(p, r, 0.5f * kExpScale);
  p = __builtin_fmaf(p, r, kExpScale);
  p = __builtin_fmaf(p, r, kExpScale);
  return rintf(ldexpf(p, (int)n));
}

// PoT: the number of bin edges base·2^j (j = 0..20) strictly below m, i.e.
// the smallest j in [0, 21] with m ≤ base·2^j (21 if none).  For m ≥ 0 and a
// normal base it follows from the float fields: with m = 1.f_m·2^e_m and
// base = 1.f_b·2^e_b, m ≤ base·2^j holds exactly when j ≥ e_m − e_b + [f_m >
// f_b]; zero and subnormal m give j ≤ 0.  Equal to the 21 compares for every
// non-negative float and every base in [2^-100, 2^100].
__device__ __forceinline__ int pot_of(float m, float base) {
  const uint32_t bm = __float_as_uint(m), bb = __float_as_uint(base);
  const int j = (int)(bm >> 23) - (int)(bb >> 23) + ((bm & 0x7FFFFFu) > (bb & 0x7FFFFFu) ? 1 : 0);
  return min(max(j, 0), kPotMax);
}

// FMDQ-INT8 code of x in a sub-channel of this PoT.
__device__ __forceinline__ int code8(float x, float inv_base, int pot) {
  const float scale = ldexpf(1.0f, kP8 - pot);   // 2^-e, e = PoT − 6
  const float r = __fmul_rn(__fmul_rn(x, inv_base), scale);
  return (int)fminf(fmaxf(rintf(r), -64.0f), 64.0f);
}

// Symmetric int8 code of x at a weight-side scale (0 where the scale is 0).
__device__ __forceinline__ int code_w(float x, float scale) {
  if (!(scale > 0.0f)) return 0;
  const double r = rint((double)x / (double)scale);
  return (int)fmin(fmax(r, -127.0), 127.0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum of v over the lanes below this one.
__device__ __forceinline__ int wave_excl_sum_i(int v) {
  const int lane = threadIdx.x & 63;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  return incl - v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
// Maximum over the 32 lanes of one half of the wave.
__device__ __forceinline__ float half_max(float v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// Planes needed for |code·2^pmax| with |code| ≤ 64.
__device__ __forceinline__ int planes_for(int pmax) {
  return 1 + (pmax >= 1 ? 1 : 0) + (pmax >= 9 ? 1 : 0) + (pmax >= 17 ? 1 : 0);
}

struct Dims {
  int64_t BH;
  int32_t heads, L, d, dp, nb;
};

Dims dims_of(const dstar_sar_params* p) {
  Dims m;
  m.BH = (int64_t)p->batch * p->heads;
  m.heads = p->heads;
  m.L = p->tokens;
  m.d = p->head_dim;
  m.dp = (p->head_dim + DSTAR_SAR_PAD - 1) / DSTAR_SAR_PAD * DSTAR_SAR_PAD;
  m.nb = p->tokens / kBlock;
  return m;
}

// ---------------------------------------------------------------- quantizers

__global__ __launch_bounds__(kThreads) void qquant_kernel(const float* q, int8_t* qc, uint8_t* qpot, Dims m,
                                                          float base, float inv_base) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (tile >= m.BH * (m.L / kTile)) return;
  const int64_t row0 = tile * kTile;            // tiles never straddle (image, head) pairs
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int c = lane + 64 * half;
    if (c >= m.dp) break;
    float x[kTile];
    float mx = 0.0f;
#pragma unroll
    for (int t = 0; t < kTile; ++t) x[t] = q[(row0 + t) * m.d + min(c, m.d - 1)];   // unconditional
#pragma unroll
    for (int t = 0; t < kTile; ++t) {
      x[t] = c < m.d ? x[t] : 0.0f;
      mx = fmaxf(mx, fabsf(x[t]));
    }
    const int pot = pot_of(mx, base);
#pragma unroll
    for (int t = 0; t < kTile; ++t) qc[(row0 + t) * m.dp + c] = (int8_t)code8(x[t], inv_base, pot);
    qpot[tile * m.dp + c] = (uint8_t)pot;
  }
}

// One wave per kKRows consecutive key rows: every row's loads are issued
// before the first maximum is taken (one row per wave left each wave with a
// single row's latency to hide).
constexpr int kKRows = 8;
__global__ __launch_bounds__(kThreads) void kquant_kernel(const float* k, int8_t* kc, float* ks, Dims m) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * kKRows;
  const int64_t rows = m.BH * m.L;
  if (row0 >= rows) return;
  float x0[kKRows], x1[kKRows];
#pragma unroll
  for (int i = 0; i < kKRows; ++i) {
    const int64_t row = min(row0 + i, rows - 1);   // rows past the end are never stored
    x0[i] = lane < m.d ? k[row * m.d + lane] : 0.0f;
    x1[i] = lane + 64 < m.d ? k[row * m.d + lane + 64] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < kKRows; ++i) {
    const int64_t row = row0 + i;
    if (row >= rows) break;
    const float amax = wave_max(fmaxf(fabsf(x0[i]), fabsf(x1[i])));
    const float s = (float)((double)amax / 127.0);
    if (lane < m.dp) kc[row * m.dp + lane] = (int8_t)code_w(x0[i], s);
    if (lane + 64 < m.dp) kc[row * m.dp + lane + 64] = (int8_t)code_w(x1[i], s);
    if (lane == 0) ks[row] = s;
  }
}

// Eight lanes per key row when d is a multiple of 4 and K is 16-byte aligned:
// lane j of a row's group holds channels [j·W, j·W + W) (W = dp/8, so the
// group covers the padded row), read as 16-byte pieces and written back as W
// code bytes; the row's maximum takes three shuffles within the group.  A
// wave takes 8·kKSets rows, all their loads in flight together.  Same codes
// and scales as kquant_kernel.
constexpr int kKSets = 2;
template <int W>
__global__ __launch_bounds__(kThreads) void kquant8_kernel(const float* k, int8_t* kc, float* ks, Dims m) {
  constexpr int NV = W / 4;
  const int lane = threadIdx.x & 63, j = lane & 7, grp = lane >> 3;
  const int64_t rows = m.BH * m.L;
  const int64_t row0 = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * (8 * kKSets);
  if (row0 >= rows) return;
  float4 x[kKSets][NV];
#pragma unroll
  for (int st = 0; st < kKSets; ++st) {
    const int64_t row = min(row0 + 8 * st + grp, rows - 1);   // rows past the end are never stored
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = j * W + 4 * i;
      x[st][i] = *reinterpret_cast<const float4*>(k + row * m.d + (c < m.d ? c : 0));   // unconditional
    }
  }
#pragma unroll
  for (int st = 0; st < kKSets; ++st) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (j * W + 4 * i >= m.d) x[st][i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      mx = fmaxf(fmaxf(mx, fmaxf(fabsf(x[st][i].x), fabsf(x[st][i].y))), fmaxf(fabsf(x[st][i].z), fabsf(x[st][i].w)));
    mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    const float sc = (float)((double)mx / 127.0);
    const int64_t row = row0 + 8 * st + grp;
    if (row < rows) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(kc + row * m.dp + j * W);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const float4 v = x[st][i];
        dst[i] = ((uint32_t)code_w(v.x, sc) & 0xFFu) | (((uint32_t)code_w(v.y, sc) & 0xFFu) << 8) |
                 (((uint32_t)code_w(v.z, sc) & 0xFFu) << 16) | (((uint32_t)code_w(v.w, sc) & 0xFFu) << 24);
      }
      if (j == 0) ks[row] = sc;
    }
  }
}

__global__ void vinit_kernel(uint32_t* bits, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) bits[i] = 0u;
}

// Partial column maxima of one 256-row chunk, lowered into the maximum's bits
// (non-negative floats order like their bit patterns).
constexpr int kVChunk = 256;
__global__ __launch_bounds__(kThreads) void vmax_kernel(const float* v, uint32_t* vmax, Dims m, int chunks) {
  __shared__ float part[kWaves][128];
  const int lane = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int64_t bh = blockIdx.x / chunks;
  const int ch = blockIdx.x % chunks;
  const int r_end = min(m.L, (ch + 1) * kVChunk);
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int c = lane + 64 * cc;
    float mx = 0.0f;
    if (c < m.d) {
      // sixteen rows' loads in flight per step
      for (int r = ch * kVChunk + rg; r < r_end; r += 16 * kWaves) {
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)   // unconditional (clamped row), so all are in flight
          x[i] = v[(bh * m.L + min(r + i * kWaves, r_end - 1)) * m.d + c];
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, r + i * kWaves < r_end ? fabsf(x[i]) : 0.0f);
      }
    }
    part[rg][c] = mx;
  }
  __syncthreads();
  const int c = threadIdx.x;
  if (c < m.d) {
    float mx = part[0][c];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, part[w][c]);
    if (mx > 0.0f) atomicMax(vmax + bh * m.d + c, __float_as_uint(mx));
  }
}

// Codes of one 64-key chunk, written channel-major: thread → (channel,
// 16 consecutive keys), one 16-byte store.
__global__ __launch_bounds__(kThreads) void vquant_kernel(const float* v, const uint32_t* vmax, int8_t* vct,
                                                          Dims m) {
  const int kchunks = m.L / 64;
  const int64_t bh = blockIdx.x / kchunks;
  const int kc = blockIdx.x % kchunks;
  const int q4 = threadIdx.x & 3;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int c = (threadIdx.x >> 2) + 64 * pass;
    if (c >= m.dp) break;
    const float s = c < m.d ? (float)((double)__uint_as_float(vmax[bh * m.d + c]) / 127.0) : 0.0f;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)   // unconditional (clamped channel; s = 0 gives code 0 there)
      x[i] = v[(bh * m.L + (int64_t)kc * 64 + 16 * q4 + i) * m.d + min(c, m.d - 1)];
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i / 4] |= ((uint32_t)code_w(x[i], s) & 0xFFu) << (8 * (i % 4));
    *reinterpret_cast<uint4*>(vct + (bh * m.dp + c) * m.L + (int64_t)kc * 64 + 16 * q4) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__global__ void vscale_kernel(uint32_t* bits, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) reinterpret_cast<float*>(bits)[i] = (float)((double)__uint_as_float(bits[i]) / 127.0);
}

// ---------------------------------------------------------------- scores

struct ScoreArgs {
  Dims m;
  int32_t B, nnz;
  const int32_t* row_ptr;
  const int32_t* cols;
  const int8_t* qc;
  const uint8_t* qpot;
  const int8_t* kc;
  const float* ks;
  int8_t* pc;
  uint8_t* ppot;
  double g;          // (base_q·2^-6)·sm_scale
  float base_p, inv_base_p;
  int32_t clip_p;    // base_p·2^21 < 1: P codes can exceed 64 and are clipped
};

// Kept-block column at a wave-uniform index.  The mask is read-only for the
// whole launch, so it is read through the constant address space: the load
// becomes a scalar load, which the vector-memory counter does not include
// (a vector load here made every iteration wait for all loads in flight).
typedef __attribute__((address_space(4))) const int32_t* const_i32_ptr;
__device__ __forceinline__ int mask_col(const int32_t* cols, int j) { return ((const_i32_ptr)cols)[j]; }

// Kept-block range of a query block, clamped to [0, nnz].
__device__ __forceinline__ void block_range(const int32_t* row_ptr, int64_t r, int32_t nnz, int& j0, int& j1) {
  j0 = min(max(row_ptr[r], 0), nnz);
  j1 = min(max(row_ptr[r + 1], j0), nnz);
}

constexpr int kOrderPerLane = 16;                  // counts a lane holds
constexpr int kOrderMax = 64 * kOrderPerLane;      // (head, query block) pairs

// The (head, query block) pair at position `rank` when all U pairs are taken
// in descending order of their kept-block counts, ties in index order; the
// result is wave-uniform.  Lane l holds the counts of pairs 16·l .. 16·l+15
// (−1 past U).  The count c at that position is the largest c with at least
// rank + 1 pairs counting c or more (a binary search over c); the pair is
// then the k-th pair counting exactly c, k = rank − #(counts above c).
// U ≤ kOrderMax.
__device__ int pair_by_rank(const int32_t* row_ptr, int32_t nnz, int U, int rank) {
  const int lane = threadIdx.x & 63;
  const int u0 = lane * kOrderPerLane;
  int rp[kOrderPerLane + 1];
#pragma unroll
  for (int i = 0; i <= kOrderPerLane; ++i) rp[i] = row_ptr[min(u0 + i, U)];   // all in flight at once
  int cnt[kOrderPerLane];
  int cmax = 0;
#pragma unroll
  for (int i = 0; i < kOrderPerLane; ++i) {
    const int j0 = min(max(rp[i], 0), nnz);
    const int j1 = min(max(rp[i + 1], j0), nnz);
    cnt[i] = u0 + i < U ? j1 - j0 : -1;
    cmax = max(cmax, cnt[i]);
  }
  cmax = __builtin_amdgcn_readfirstlane(wave_max_i(cmax));
  auto count_at_least = [&](int c) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < kOrderPerLane; ++i) n += cnt[i] >= c ? 1 : 0;
    return __builtin_amdgcn_readfirstlane(wave_sum_i(n));
  };
  int lo = 0, hi = cmax;          // count_at_least(lo) = U > rank
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (count_at_least(mid) > rank) lo = mid;
    else hi = mid - 1;
  }
  int k = rank - (lo < cmax ? count_at_least(lo + 1) : 0);
  int m = 0;
#pragma unroll
  for (int i = 0; i < kOrderPerLane; ++i) m += cnt[i] == lo ? 1 : 0;
  const int before = wave_excl_sum_i(m);
  int pick = 0x7FFFFFFF;
  if (before <= k && k < before + m) {
    int t = k - before;
#pragma unroll
    for (int i = 0; i < kOrderPerLane; ++i) {
      if (cnt[i] == lo) {
        if (t == 0) pick = u0 + i;
        --t;
      }
    }
  }
  return __builtin_amdgcn_readfirstlane(min(wave_min_i(pick), U - 1));
}

// The tile of wave g of the scores kernel: g / (2·batch) is the rank of its
// (head, query block) pair in the order above, so waves with the most kept
// blocks start first and the shortest fill in at the end (longest processing
// time first; the grid runs two waves per SIMD over several rounds);
// g % (2·batch) picks the image and which of the block's two token tiles.
// Pairs beyond kOrderMax keep index order.
struct TileWork {
  int64_t bh;
  int tau, b, h, qb, half;
};
__device__ __forceinline__ TileWork tile_work(const Dims& m, const int32_t* row_ptr, int32_t nnz, int B,
                                              int64_t g) {
  const int U = m.heads * m.nb;
  const int per = 2 * B;
  const int rank = (int)(g / per), sub = (int)(g % per);
  const int pair = U <= kOrderMax ? pair_by_rank(row_ptr, nnz, U, rank) : rank;
  TileWork w;
  w.h = pair / m.nb;
  w.qb = pair % m.nb;
  w.b = sub >> 1;
  w.half = sub & 1;
  w.bh = (int64_t)w.b * m.heads + w.h;
  w.tau = 2 * w.qb + w.half;
  return w;
}

// Digit planes 0..NP-1 of 16 values a_i = code_i·2^pot_i (codes: signed
// bytes of cw, PoTs: bytes of pw); dig[j] holds digit j of the 16 values, 4
// per int.  The caller guarantees that the higher digits are 0.  Adding
// Σ_j 128·256^j to a makes every digit non-negative (d_j + 128 in [0, 255]),
// so the bytes of a + 0x80808080, each XORed with 0x80, are the signed
// digits of a (|a| ≤ 2^27); a 4 × 4 byte transpose then gathers digit j of
// four values into one word.
template <int NP>
__device__ __forceinline__ void digits_np(const v4i cw, const v4i pw, v4i (&dig)[NP]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int code = (int)(int8_t)(((uint32_t)cw[w] >> (8 * i)) & 0xFFu);
      const int pot = (int)(((uint32_t)pw[w] >> (8 * i)) & 0xFFu);
      d[i] = ((uint32_t)(code * (1 << pot)) + 0x80808080u) ^ 0x80808080u;
    }
    // d[i] = bytes (d0, d1, d2, d3) of value i → plane words
    const uint32_t a0 = __builtin_amdgcn_perm(d[1], d[0], 0x05010400u);
    const uint32_t a1 = __builtin_amdgcn_perm(d[1], d[0], 0x07030602u);
    const uint32_t b0 = __builtin_amdgcn_perm(d[3], d[2], 0x05010400u);
    const uint32_t b1 = __builtin_amdgcn_perm(d[3], d[2], 0x07030602u);
    const uint32_t pl[4] = {__builtin_amdgcn_perm(b0, a0, 0x05040100u), __builtin_amdgcn_perm(b0, a0, 0x07060302u),
                            __builtin_amdgcn_perm(b1, a1, 0x05040100u), __builtin_amdgcn_perm(b1, a1, 0x07060302u)};
#pragma unroll
    for (int j = 0; j < NP; ++j) dig[j][w] = (int)pl[j];
  }
}

// Largest PoT byte of a 16-byte vector.
__device__ __forceinline__ int max_pot16(const v4i pw) {
  int m = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, (int)(((uint32_t)pw[w] >> (8 * i)) & 0xFFu));
  return m;
}

// Logits z of one 32-key column tile of a kept block for the wave's 32 rows:
// z[r] at row 8·(r/4) + 4·(lane/32) + r%4 of the tile and key lane%32 of the
// column tile.  The exact integer score is Σ_j 2^(8j)·(digit plane j · K);
// with two planes every partial sum and the total stay below 2^30, so int32
// holds it exactly, otherwise the planes are combined in int64.
template <int NKS, int NP>
__device__ __forceinline__ void tile_logits(const v4i (&A)[NKS][NP], const v4i (&B)[NKS], double f, float (&z)[16]) {
  if constexpr (NP <= 2) {
    v16i acc[NP];
#pragma unroll
    for (int jp = 0; jp < NP; ++jp) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[jp][r] = 0;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc[jp] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[ks][jp], B[ks], acc[jp], 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int s = NP == 2 ? acc[0][r] + acc[1][r] * 256 : acc[0][r];
      z[r] = (float)((double)s * f);
    }
  } else {
    // one plane at a time into an int64 sum (fewer live registers)
    int64_t s[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0;
#pragma unroll
    for (int jp = 0; jp < NP; ++jp) {
      v16i acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[ks][jp], B[ks], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] += (int64_t)acc[r] * ((int64_t)1 << (8 * jp));
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = (float)((double)s[r] * f);
  }
}

__device__ __forceinline__ double half_sum_d(double v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One sweep over the kept blocks [j0, j1) of the wave's query block: the
// logits of every 32-key column tile are handed to fn(j, ct, z).  With two
// digit planes the K fragments and scales of block j+1 are loaded while
// block j is computed (with four there are no registers left for that).
template <int NKS, int NP, typename F>
__device__ __forceinline__ void sweep_blocks(const ScoreArgs& a, int64_t bh, int j0, int j1,
                                             const v4i (&A)[NKS][NP], F&& fn) {
  const int lane = threadIdx.x & 63, li = lane & 31, hi = lane >> 5;
  const int8_t* kbh = a.kc + bh * a.m.L * (int64_t)a.m.dp + (int64_t)li * a.m.dp + 16 * hi;
  const float* sbh = a.ks + bh * a.m.L + li;
  v4i Bn[2][NKS];
  float sn[2];
  auto fetch = [&](int j) {
    int kb = mask_col(a.cols, j);
    kb = (kb < 0 || kb >= a.m.nb) ? 0 : kb;     // skipped below; any block in range
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        Bn[ct][ks] = *reinterpret_cast<const v4i*>(kbh + (int64_t)(kb * kBlock + 32 * ct) * a.m.dp + 32 * ks);
      sn[ct] = sbh[kb * kBlock + 32 * ct];
    }
  };
  constexpr bool kPrefetch = NP <= 2;
  if (kPrefetch) fetch(j0);
  for (int j = j0; j < j1; ++j) {
    const int kb = mask_col(a.cols, j);
    if (!kPrefetch) fetch(j);
    v4i B[2][NKS];
    float sc[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      sc[ct] = sn[ct];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) B[ct][ks] = Bn[ct][ks];
    }
    if (kPrefetch) {
      fetch(min(j + 1, j1 - 1));   // unconditional: a constant load count
      __asm__ __volatile__("" ::: "memory");   // issue it here, not where it is used
    }
    if (kb < 0 || kb >= a.m.nb) continue;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float z[16];
      tile_logits<NKS, NP>(A, B[ct], (double)sc[ct] * a.g, z);
      fn(j, ct, z);
    }
  }
}

// The low byte of rint(r) for r in [0, 2^22]: r + 2^23 rounds to the integer
// nearest r (ties to even) in the low mantissa bits, and a byte store keeps
// those bits.
__device__ __forceinline__ int8_t rint_byte(float r) {
  return (int8_t)__float_as_uint(__fadd_rn(r, 0x1p23f));
}

// Sweeps 2 and 3 of one 32-row query tile, given the row maxima of the
// logits: exact sums of the fixed-point exponentials E (ΣE ≥ 2^36, as the
// row maximum gives E = 2^36), then P = fl32(f64(E)·(1/f64(ΣE))) in [0, 1],
// its FMDQ-INT8 codes per (tile, key) sub-channel and the cache.  kClamp
// selects the exponential with the cut-off clamp (logit spreads beyond
// kXSafe).  Codes: q = rint(fl32(fl32(P·inv_base)·2^(6−PoT))), clipped to
// 64.  The power of two is folded into inv_base once per column; that product
// is exact for bases in [2^-100, 2^100], and fl32(P·(inv_base·2^(6−PoT))) is
// then the same float while both forms are normal (otherwise both are below
// 2^-126 and give 0).  P ≥ 0 gives q ≥ 0, and P ≤ max P ≤ base·2^PoT keeps q
// ≤ 64 unless the PoT saturates, which needs base·2^21 < 1 (P ≤ 1): only
// then is the clip applied (a.clip_p).
template <int NKS, int NP, bool kClamp>
__device__ __forceinline__ void scores_sweeps23(const ScoreArgs& a, int64_t bh, int b, int half, int j0, int j1,
                                                const v4i (&A)[NKS][NP], const float (&mrow)[16]) {
  const int lane = threadIdx.x & 63, li = lane & 31, hi = lane >> 5;
  double inv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) inv[r] = 0.0;
  sweep_blocks<NKS, NP>(a, bh, j0, j1, A, [&](int, int, const float (&z)[16]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) inv[r] += (double)exp_fixed<kClamp>(__fsub_rn(z[r], mrow[r]));
  });
#pragma unroll
  for (int r = 0; r < 16; ++r) inv[r] = 1.0 / half_sum_d(inv[r]);

  sweep_blocks<NKS, NP>(a, bh, j0, j1, A, [&](int j, int ct, const float (&z)[16]) {
    const int64_t blk = (int64_t)b * a.nnz + j;
    float P[16];
    float mx = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      P[r] = (float)((double)exp_fixed<kClamp>(__fsub_rn(z[r], mrow[r])) * inv[r]);
      mx = fmaxf(mx, P[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));    // the other 16 rows of the column
    const int pot = pot_of(mx, a.base_p);
    const float ib = ldexpf(a.inv_base_p, kP8 - pot);
    int8_t* dst = a.pc + (blk * kBlock + 32 * half) * kBlock + 32 * ct + li;
    if (a.clip_p) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dst[(8 * (r >> 2) + 4 * hi + (r & 3)) * kBlock] = rint_byte(fminf(__fmul_rn(P[r], ib), 64.0f));
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dst[(8 * (r >> 2) + 4 * hi + (r & 3)) * kBlock] = rint_byte(__fmul_rn(P[r], ib));
    }
    if (hi == 0) a.ppot[(blk * 2 + half) * kBlock + 32 * ct + li] = (uint8_t)pot;
  });
}

// The three sweeps of one 32-row query tile (a wave) with NP digit planes of
// a_Q: row maxima of the logits (and the wave's smallest logit), then sweeps
// 2 and 3.  Exponent arguments x = z − max z stay within [−kXSafe, 0] when
// the wave's logits span at most kXSafe, and then need no clamp.
template <int NKS, int NP>
__device__ __forceinline__ void scores_tile(const ScoreArgs& a, int64_t bh, int b, int half, int j0, int j1,
                                            const v4i (&cw)[NKS], const v4i (&pw)[NKS]) {
  v4i A[NKS][NP];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) digits_np<NP>(cw[ks], pw[ks], A[ks]);

  float mrow[16];
  float zlo = INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) mrow[r] = -INFINITY;
  sweep_blocks<NKS, NP>(a, bh, j0, j1, A, [&](int, int, const float (&z)[16]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      mrow[r] = fmaxf(mrow[r], z[r]);
      zlo = fminf(zlo, z[r]);
    }
  });
  float mhi = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    mrow[r] = half_max(mrow[r]);
    mhi = fmaxf(mhi, mrow[r]);
  }
  mhi = wave_max(mhi);
  zlo = wave_min(zlo);
  // wave-uniform: a scalar branch, not two masked bodies
  const int wide = __builtin_amdgcn_readfirstlane(mhi - zlo <= kXSafe ? 0 : 1);
  if (wide)
    scores_sweeps23<NKS, NP, true>(a, bh, b, half, j0, j1, A, mrow);
  else
    scores_sweeps23<NKS, NP, false>(a, bh, b, half, j0, j1, A, mrow);
}

// One wave per (image·head, 32-row token tile); NKS = dp/32 k-steps.  Two
// waves per SIMD: the digit planes of a_Q the tile needs (two unless some
// PoT exceeds 8) select the instantiation, so the common case keeps few
// registers.
template <int NKS>
__global__ __launch_bounds__(kThreads, 2) void scores_kernel(ScoreArgs a) {
  const int lane = threadIdx.x & 63, li = lane & 31, hi = lane >> 5;
  const int tpb = a.m.L / kTile;
  // wave-uniform (readfirstlane): the index and mask loads below become
  // scalar loads, which the vector-load counts do not include
  const int64_t tile = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWaves + (threadIdx.x >> 6)));
  if (tile >= a.m.BH * tpb) return;
  const TileWork w = tile_work(a.m, a.row_ptr, a.nnz, a.B, tile);
  const int64_t bh = w.bh;
  const int tau = w.tau, b = w.b, half = w.half;
  int j0, j1;
  block_range(a.row_ptr, (int64_t)w.h * a.m.nb + w.qb, a.nnz, j0, j1);
  if (j0 >= j1) return;

  v4i cw[NKS], pw[NKS];
  int pmax = 0;
  {
    const int8_t* qrow = a.qc + (bh * a.m.L + (int64_t)tau * kTile + li) * a.m.dp;
    const uint8_t* prow = a.qpot + (bh * tpb + tau) * a.m.dp;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      cw[ks] = *reinterpret_cast<const v4i*>(qrow + 32 * ks + 16 * hi);
      pw[ks] = *reinterpret_cast<const v4i*>(prow + 32 * ks + 16 * hi);
      pmax = max(pmax, max_pot16(pw[ks]));
    }
  }
  if (planes_for(wave_max_i(pmax)) <= 2)
    scores_tile<NKS, 2>(a, bh, b, half, j0, j1, cw, pw);
  else
    scores_tile<NKS, kPlanes>(a, bh, b, half, j0, j1, cw, pw);
}

// ---------------------------------------------------------------- P·V

struct PvArgs {
  Dims m;
  int32_t B, nnz;
  const int32_t* row_ptr;
  const int32_t* cols;
  const int8_t* pc;
  const uint8_t* ppot;
  const int8_t* vct;
  const float* vscale;
  float* out;
  double hp;         // base_p·2^-6
};

// One pass over the kept blocks of the wave's query block for the column
// tiles ct0 .. ct0+CG-1 (those below ncg): a_P is split into NP digit planes
// (NP covers every kept block's largest PoT); each (column tile, plane) keeps
// one int32 MFMA accumulator over all kept keys.  |digit| ≤ 128, |V code| ≤
// 127 and at most 2^16 keys, so each stays below 2^31 and is exact; the
// planes are combined in int64 once, at the end.  The P codes and PoTs of
// block j+1 are loaded while block j is multiplied.
template <int CG, int NP>
__device__ __forceinline__ void pv_pass(const PvArgs& a, int64_t bh, int tau, int b, int half, int j0, int j1,
                                        int ct0, int ncg) {
  const int lane = threadIdx.x & 63, li = lane & 31, hi = lane >> 5;
  v16i acc[CG][NP];
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int jp = 0; jp < NP; ++jp)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][jp][r] = 0;

  v4i cn[2], pn[2];
  auto fetch = [&](int j) {
    const int64_t blk = (int64_t)b * a.nnz + j;
    const int8_t* prow = a.pc + (blk * kBlock + 32 * half + li) * kBlock + 16 * hi;
    const uint8_t* pp = a.ppot + (blk * 2 + half) * kBlock + 16 * hi;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      cn[ks] = *reinterpret_cast<const v4i*>(prow + 32 * ks);
      pn[ks] = *reinterpret_cast<const v4i*>(pp + 32 * ks);
    }
  };
  const int8_t* vbh = a.vct + (bh * a.m.dp + li) * (int64_t)a.m.L + 16 * hi;
  if (j0 < j1) fetch(j0);
  for (int j = j0; j < j1; ++j) {
    const int kb = mask_col(a.cols, j);
    const bool valid = kb >= 0 && kb < a.m.nb;
    const v4i cw0 = cn[0], cw1 = cn[1], pw0 = pn[0], pw1 = pn[1];
    // V fragments of this block first, then the next block's P: vector loads
    // complete in order, so waiting for V leaves the prefetch in flight.
    v4i Bv[CG][2];
    const int kbc = valid ? kb : 0;
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      const int8_t* vrow = vbh + (int64_t)(32 * (ct0 + min(c, ncg - 1))) * a.m.L + (int64_t)kbc * kBlock;
      Bv[c][0] = *reinterpret_cast<const v4i*>(vrow);
      Bv[c][1] = *reinterpret_cast<const v4i*>(vrow + 32);
    }
    __asm__ __volatile__("" ::: "memory");
    fetch(min(j + 1, j1 - 1));   // unconditional: a constant load count
    __asm__ __volatile__("" ::: "memory");
    if (!valid) continue;
    v4i A0[NP], A1[NP];
    digits_np<NP>(cw0, pw0, A0);
    digits_np<NP>(cw1, pw1, A1);
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      if (c < ncg) {
#pragma unroll
        for (int jp = 0; jp < NP; ++jp) {
          acc[c][jp] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A0[jp], Bv[c][0], acc[c][jp], 0, 0, 0);
          acc[c][jp] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A1[jp], Bv[c][1], acc[c][jp], 0, 0, 0);
        }
      }
    }
  }

#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const int ch = 32 * (ct0 + c) + li;
    if (c < ncg && ch < a.m.d) {
      const double hc = (double)a.vscale[bh * a.m.d + ch] * a.hp;
      float* dst = a.out + (bh * a.m.L + (int64_t)tau * kTile) * a.m.d + ch;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int64_t o = 0;
#pragma unroll
        for (int jp = 0; jp < NP; ++jp) o += (int64_t)acc[c][jp][r] * ((int64_t)1 << (8 * jp));
        dst[(int64_t)(8 * (r >> 2) + 4 * hi + (r & 3)) * a.m.d] = (float)((double)o * hc);
      }
    }
  }
}

// All column tiles of one wave's rows, CG at a time.
template <int NCT, int CG, int NP>
__device__ __forceinline__ void pv_tile(const PvArgs& a, int64_t bh, int tau, int b, int half, int j0, int j1) {
#pragma unroll
  for (int ct0 = 0; ct0 < NCT; ct0 += CG) pv_pass<CG, NP>(a, bh, tau, b, half, j0, j1, ct0, min(CG, NCT - ct0));
}

// One wave per (image·head, 32-row token tile); NCT = dp/32 column tiles.
// A first pass over the kept blocks' PoTs of the tile's rows gives the digit
// planes a_P needs (P ≤ 1: three planes while every PoT ≤ 16), which select
// the instantiation; two waves per SIMD.
template <int NCT>
__global__ __launch_bounds__(kThreads, 2) void pv_kernel(PvArgs a) {
  const int lane = threadIdx.x & 63;
  const int tpb = a.m.L / kTile;
  // wave-uniform (readfirstlane): the index and mask loads below become
  // scalar loads, which the vector-load counts do not include
  // index order: a pv wave is short enough (about a third of a scores wave)
  // that the longest-first lookup costs more than it evens out
  const int64_t tile = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWaves + (threadIdx.x >> 6)));
  if (tile >= a.m.BH * tpb) return;
  const int64_t bh = tile / tpb;
  const int tau = (int)(tile % tpb);
  const int b = (int)(bh / a.m.heads), h = (int)(bh % a.m.heads);
  const int qb = tau >> 1, half = tau & 1;
  int j0, j1;
  block_range(a.row_ptr, (int64_t)h * a.m.nb + qb, a.nnz, j0, j1);

  int pmax = 0;
  for (int j = j0; j < j1; j += 8) {
    int pt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)   // eight loads in flight (indices clamped, extras ignored)
      pt[i] = a.ppot[(((int64_t)b * a.nnz + min(j + i, j1 - 1)) * 2 + half) * kBlock + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kb = a.cols[min(j + i, j1 - 1)];
      if (j + i < j1 && kb >= 0 && kb < a.m.nb) pmax = max(pmax, pt[i]);
    }
  }
  const int np = planes_for(min(wave_max_i(pmax), 31));
  if (np <= 2)
    pv_tile<NCT, (NCT < 3 ? NCT : 3), 2>(a, bh, tau, b, half, j0, j1);
  else if (np == 3)
    pv_tile<NCT, (NCT < 3 ? NCT : 3), 3>(a, bh, tau, b, half, j0, j1);
  else
    pv_tile<NCT, (NCT < 2 ? NCT : 2), kPlanes>(a, bh, tau, b, half, j0, j1);
}

// ---------------------------------------------------------------- host checks

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool base_ok(float b) { return std::isfinite(b) && b >= std::ldexp(1.0f, -100) && b <= std::ldexp(1.0f, 100); }

int check(const dstar_sar_params* p) {
  if (p == nullptr) return set_error(DSTAR_ENULL, "sar params is NULL");
  if (p->batch < 1 || p->heads < 1) return set_error(DSTAR_EINVAL, "batch = %d, heads = %d must be >= 1", p->batch, p->heads);
  if (p->tokens < kBlock || p->tokens > DSTAR_SAR_MAX_L || p->tokens % kBlock != 0)
    return set_error(DSTAR_EINVAL, "tokens = %d must be a multiple of %d in [%d, %d]", p->tokens, kBlock, kBlock,
                     DSTAR_SAR_MAX_L);
  if (p->head_dim < 1 || p->head_dim > DSTAR_SAR_MAX_D)
    return set_error(DSTAR_EINVAL, "head_dim = %d outside [1, %d]", p->head_dim, DSTAR_SAR_MAX_D);
  if (!base_ok(p->base_q) || !base_ok(p->base_p))
    return set_error(DSTAR_EINVAL, "base_q = %g / base_p = %g outside [2^-100, 2^100]", (double)p->base_q,
                     (double)p->base_p);
  if (!std::isfinite(p->sm_scale) || !(p->sm_scale > 0.0f))
    return set_error(DSTAR_EINVAL, "sm_scale = %g must be finite and > 0", (double)p->sm_scale);
  if ((int64_t)p->batch * p->heads * p->tokens > ((int64_t)1 << 31))
    return set_error(DSTAR_EINVAL, "batch·heads·tokens exceeds 2^31");
  return DSTAR_OK;
}

int check_ptrs(std::initializer_list<std::pair<const void*, size_t>> ps) {
  for (const auto& pr : ps) {
    if (pr.first == nullptr) return set_error(DSTAR_ENULL, "a required pointer is NULL");
    if (!aligned(pr.first, pr.second)) return set_error(DSTAR_EALIGN, "pointer %p not %zu-byte aligned", pr.first, pr.second);
  }
  return DSTAR_OK;
}

int check_csr(const dstar_sar_params* p, const int32_t* row_ptr, const int32_t* cols, int32_t nnz) {
  const int64_t nb = p->tokens / kBlock;
  if (nnz < 0 || nnz > (int64_t)p->heads * nb * nb)
    return set_error(DSTAR_EINVAL, "nnz = %d outside [0, heads·(L/64)^2]", nnz);
  if ((int64_t)p->batch * nnz * kBlock * kBlock > ((int64_t)1 << 40))
    return set_error(DSTAR_EINVAL, "cache too large");
  if (row_ptr == nullptr || (nnz > 0 && cols == nullptr)) return set_error(DSTAR_ENULL, "row_ptr / cols is NULL");
  if (!aligned(row_ptr, 4) || !aligned(cols, 4)) return set_error(DSTAR_EALIGN, "row_ptr / cols not 4-byte aligned");
  return DSTAR_OK;
}

unsigned waves_grid(int64_t waves) { return (unsigned)((waves + kWaves - 1) / kWaves); }

}  // namespace
}  // namespace dstar

using namespace dstar;

extern "C" {

int dstar_sar_quantize_q(const dstar_sar_params* p, const float* q, int8_t* qcodes, uint8_t* qpot, void* stream) {
  clear_error();
  if (int rc = check(p)) return rc;
  if (int rc = check_ptrs({{q, 4}, {qcodes, 16}, {qpot, 16}})) return rc;
  const Dims m = dims_of(p);
  const float inv = (float)(1.0 / (double)p->base_q);
  hipLaunchKernelGGL(qquant_kernel, dim3(waves_grid(m.BH * (m.L / kTile))), dim3(kThreads), 0, (hipStream_t)stream, q,
                     qcodes, qpot, m, p->base_q, inv);
  return check_launch("sar_quantize_q");
}

int dstar_sar_quantize_k(const dstar_sar_params* p, const float* k, int8_t* kcodes, float* kscale, void* stream) {
  clear_error();
  if (int rc = check(p)) return rc;
  if (int rc = check_ptrs({{k, 4}, {kcodes, 16}, {kscale, 4}})) return rc;
  const Dims m = dims_of(p);
  const hipStream_t s = (hipStream_t)stream;
  if (m.d % 4 == 0 && aligned(k, 16)) {
    const dim3 grid(waves_grid((m.BH * m.L + 8 * kKSets - 1) / (8 * kKSets))), block(kThreads);
    switch (m.dp / 8) {
      case 4: hipLaunchKernelGGL(kquant8_kernel<4>, grid, block, 0, s, k, kcodes, kscale, m); break;
      case 8: hipLaunchKernelGGL(kquant8_kernel<8>, grid, block, 0, s, k, kcodes, kscale, m); break;
      case 12: hipLaunchKernelGGL(kquant8_kernel<12>, grid, block, 0, s, k, kcodes, kscale, m); break;
      default: hipLaunchKernelGGL(kquant8_kernel<16>, grid, block, 0, s, k, kcodes, kscale, m); break;
    }
  } else {
    hipLaunchKernelGGL(kquant_kernel, dim3(waves_grid((m.BH * m.L + kKRows - 1) / kKRows)), dim3(kThreads), 0, s,
                       k, kcodes, kscale, m);
  }
  return check_launch("sar_quantize_k");
}

int dstar_sar_quantize_v(const dstar_sar_params* p, const float* v, int8_t* vcodes_t, float* vscale, void* stream) {
  clear_error();
  if (int rc = check(p)) return rc;
  if (int rc = check_ptrs({{v, 4}, {vcodes_t, 16}, {vscale, 4}})) return rc;
  const Dims m = dims_of(p);
  const hipStream_t s = (hipStream_t)stream;
  uint32_t* bits = reinterpret_cast<uint32_t*>(vscale);
  const int64_t n = m.BH * m.d;
  hipLaunchKernelGGL(vinit_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, bits, n);
  if (int rc = check_launch("sar_quantize_v (init)")) return rc;
  const int chunks = (m.L + kVChunk - 1) / kVChunk;
  hipLaunchKernelGGL(vmax_kernel, dim3((unsigned)(m.BH * chunks)), dim3(kThreads), 0, s, v, bits, m, chunks);
  if (int rc = check_launch("sar_quantize_v (max)")) return rc;
  hipLaunchKernelGGL(vquant_kernel, dim3((unsigned)(m.BH * (m.L / 64))), dim3(kThreads), 0, s, v, bits, vcodes_t, m);
  if (int rc = check_launch("sar_quantize_v (codes)")) return rc;
  hipLaunchKernelGGL(vscale_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, bits, n);
  return check_launch("sar_quantize_v (scale)");
}

int dstar_sar_scores(const dstar_sar_params* p, const int32_t* row_ptr, const int32_t* cols, int32_t nnz,
                     const int8_t* qcodes, const uint8_t* qpot, const int8_t* kcodes, const float* kscale,
                     int8_t* pcodes, uint8_t* ppot, void* stream) {
  clear_error();
  if (int rc = check(p)) return rc;
  if (int rc = check_csr(p, row_ptr, cols, nnz)) return rc;
  if (int rc = check_ptrs({{qcodes, 16}, {qpot, 16}, {kcodes, 16}, {kscale, 4}})) return rc;
  if (nnz > 0)
    if (int rc = check_ptrs({{pcodes, 16}, {ppot, 16}})) return rc;
  ScoreArgs a;
  a.m = dims_of(p);
  a.B = p->batch;
  a.nnz = nnz;
  a.row_ptr = row_ptr;
  a.cols = cols;
  a.qc = qcodes;
  a.qpot = qpot;
  a.kc = kcodes;
  a.ks = kscale;
  a.pc = pcodes;
  a.ppot = ppot;
  a.g = ((double)p->base_q * 0x1p-6) * (double)p->sm_scale;
  a.base_p = p->base_p;
  a.inv_base_p = (float)(1.0 / (double)p->base_p);
  a.clip_p = (double)p->base_p * 0x1p21 < 1.0 ? 1 : 0;
  if (nnz == 0) return DSTAR_OK;
  const dim3 grid(waves_grid(a.m.BH * (a.m.L / kTile)));
  const hipStream_t s = (hipStream_t)stream;
  switch (a.m.dp / 32) {
    case 1: hipLaunchKernelGGL(scores_kernel<1>, grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(scores_kernel<2>, grid, dim3(kThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL(scores_kernel<3>, grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(scores_kernel<4>, grid, dim3(kThreads), 0, s, a); break;
  }
  return check_launch("sar_scores");
}

int dstar_sar_pv(const dstar_sar_params* p, const int32_t* row_ptr, const int32_t* cols, int32_t nnz,
                 const int8_t* pcodes, const uint8_t* ppot, const int8_t* vcodes_t, const float* vscale, float* out,
                 void* stream) {
  clear_error();
  if (int rc = check(p)) return rc;
  if (int rc = check_csr(p, row_ptr, cols, nnz)) return rc;
  if (int rc = check_ptrs({{vcodes_t, 16}, {vscale, 4}, {out, 4}})) return rc;
  if (nnz > 0)
    if (int rc = check_ptrs({{pcodes, 16}, {ppot, 16}})) return rc;
  PvArgs a;
  a.m = dims_of(p);
  a.B = p->batch;
  a.nnz = nnz;
  a.row_ptr = row_ptr;
  a.cols = cols;
  a.pc = pcodes;
  a.ppot = ppot;
  a.vct = vcodes_t;
  a.vscale = vscale;
  a.out = out;
  a.hp = (double)p->base_p * 0x1p-6;
  const dim3 grid(waves_grid(a.m.BH * (a.m.L / kTile)));
  const hipStream_t s = (hipStream_t)stream;
  switch (a.m.dp / 32) {
    case 1: hipLaunchKernelGGL(pv_kernel<1>, grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(pv_kernel<2>, grid, dim3(kThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL(pv_kernel<3>, grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(pv_kernel<4>, grid, dim3(kThreads), 0, s, a); break;
  }
  return check_launch("sar_pv");
}

}  // extern "C"
