// Sparse Attention Reuse with FMDQ-INT8 operands (DSTAR, arXiv 2607.15846:
// §3.2 "Sparse Attention Reuse", Fig. 8; §4.3 "Attention Operation", Fig. 13).
//
// Kernels:
//   qquant  FMDQ-INT8 of Q: one wave per 32-row token tile, a lane per channel
//           (two channel passes), the tile's rows streamed with coalesced loads.
//   kquant  int8 of K with a scale per key: one wave per key row.
//   vquant  int8 of V with a scale per channel: a column-maximum pass (partial
//           maxima of 256-row chunks lowered into the scale buffer by atomic
//           max on the float bits), a quantize pass that writes the codes
//           channel-major, and a pass that turns the maxima into scales.
//   scores  cached step: one wave per (image·head, 32-row token tile); three
//           sweeps over the kept key blocks of its query block (row maximum of
//           the logits, sum of the fixed-point exponentials, then P and its
//           FMDQ-INT8 codes), each recomputing the exact integer scores.
//   pv      cached and reused steps: one wave per (image·head, token tile),
//           int64 accumulators of the exact O_int over the kept key blocks.
//
// Exact integer products on int8 MFMAs.  An FMDQ operand value in integer
// units is a = code·2^PoT (|code| ≤ 64, PoT ≤ 21, so |a| ≤ 2^27).  It is split
// into signed base-256 digits a = Σ_j 2^(8j)·d_j (d_j in [-128, 127]); each
// digit plane is an int8 matrix, and one v_mfma_i32_32x32x32_i8 chain per
// plane gives an exact int32 partial product (|Σ| ≤ 128·127·128 < 2^22) that
// is shifted into an int64 sum.  The planes a tile needs follow from its
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
constexpr int kMaxKs = DSTAR_SAR_MAX_D / 32;   // k-steps over the head channels
constexpr int kPlanes = 4;                     // digit planes of |a| ≤ 2^27
constexpr int kP8 = 6;                         // log2 of the 8-bit ceiling 64
constexpr int kPotMax = DSTAR_FMDQ_POT_MAX;    // 21
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// exp32 constants, float32 (hex literals so that both implementations start
// from the same bits): log2(e); ln 2 = LN2_HI + LN2_LO with LN2_HI = 355/512,
// whose product with the small integer n is exact; Taylor coefficients of e^r
// from 1/7! down to 1.
constexpr float kLog2e = 0x1.715476p+0f;
constexpr float kLn2Hi = 0x1.63p-1f;
constexpr float kLn2Lo = -0x1.bd0106p-13f;
constexpr float kExpXMin = -26.0f;

__device__ __forceinline__ float exp32(float x) {
  if (x < kExpXMin) return 0.0f;
  const float n = rintf(__fmul_rn(x, kLog2e));
  const float r = __fsub_rn(__fsub_rn(x, __fmul_rn(n, kLn2Hi)), __fmul_rn(n, kLn2Lo));
  float p = 0x1.a01a02p-13f;                       // 1/5040
  p = __fadd_rn(__fmul_rn(p, r), 0x1.6c16c2p-10f);  // 1/720
  p = __fadd_rn(__fmul_rn(p, r), 0x1.111112p-7f);   // 1/120
  p = __fadd_rn(__fmul_rn(p, r), 0x1.555556p-5f);   // 1/24
  p = __fadd_rn(__fmul_rn(p, r), 0x1.555556p-3f);   // 1/6
  p = __fadd_rn(__fmul_rn(p, r), 0.5f);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  return ldexpf(p, (int)n);
}

// E = rint(exp32(x)·2^36): e ≤ 1, so the scaled value is at most 2^36 and
// converts to int64 exactly.
__device__ __forceinline__ int64_t exp_fixed(float x) {
  return (int64_t)rintf(ldexpf(exp32(x), DSTAR_SAR_EXP_FRAC));
}

// PoT: the number of bin edges base·2^j (j = 0..20) strictly below m.
__device__ __forceinline__ int pot_of(float m, float base) {
  int pot = 0;
#pragma unroll
  for (int j = 0; j < kPotMax; ++j) pot += (m > ldexpf(base, j)) ? 1 : 0;
  return pot;
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
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
// Maximum / int64 sum over the 32 lanes of one half of the wave.
__device__ __forceinline__ float half_max(float v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int64_t half_sum(int64_t v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) {
    const int lo = __shfl_xor((int)(uint32_t)(uint64_t)v, o, 64);
    const int hi = __shfl_xor((int)(uint32_t)((uint64_t)v >> 32), o, 64);
    v += (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
  }
  return v;
}

// Planes needed for |code·2^pmax| with |code| ≤ 64.
__device__ __forceinline__ int planes_for(int pmax) {
  return 1 + (pmax >= 1 ? 1 : 0) + (pmax >= 9 ? 1 : 0) + (pmax >= 17 ? 1 : 0);
}

// Digit planes of 16 values a_i = code_i·2^pot_i (codes: signed bytes of cw,
// PoTs: bytes of pw); dig[j] holds digit j of the 16 values, 4 per int.
// Returns the largest PoT seen.
__device__ __forceinline__ int digits16(const v4i cw, const v4i pw, v4i (&dig)[kPlanes]) {
  int pmax = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t o[kPlanes] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int code = (int)(int8_t)(((uint32_t)cw[w] >> (8 * i)) & 0xFFu);
      const int pot = (int)(((uint32_t)pw[w] >> (8 * i)) & 0xFFu);
      pmax = max(pmax, pot);
      int a = code * (1 << pot);
#pragma unroll
      for (int j = 0; j < kPlanes; ++j) {
        const int dj = (int)(int8_t)(a & 0xFF);
        o[j] |= ((uint32_t)dj & 0xFFu) << (8 * i);
        a = (a - dj) >> 8;   // exact: a − dj is a multiple of 256
      }
    }
#pragma unroll
    for (int j = 0; j < kPlanes; ++j) dig[j][w] = (int)o[j];
  }
  return pmax;
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
    for (int t = 0; t < kTile; ++t) {
      x[t] = c < m.d ? q[(row0 + t) * m.d + c] : 0.0f;
      mx = fmaxf(mx, fabsf(x[t]));
    }
    const int pot = pot_of(mx, base);
#pragma unroll
    for (int t = 0; t < kTile; ++t) qc[(row0 + t) * m.dp + c] = (int8_t)code8(x[t], inv_base, pot);
    qpot[tile * m.dp + c] = (uint8_t)pot;
  }
}

__global__ __launch_bounds__(kThreads) void kquant_kernel(const float* k, int8_t* kc, float* ks, Dims m) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= m.BH * m.L) return;
  const float x0 = lane < m.d ? k[row * m.d + lane] : 0.0f;
  const float x1 = lane + 64 < m.d ? k[row * m.d + lane + 64] : 0.0f;
  const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float s = (float)((double)amax / 127.0);
  if (lane < m.dp) kc[row * m.dp + lane] = (int8_t)code_w(x0, s);
  if (lane + 64 < m.dp) kc[row * m.dp + lane + 64] = (int8_t)code_w(x1, s);
  if (lane == 0) ks[row] = s;
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
    if (c < m.d)
      for (int r = ch * kVChunk + rg; r < r_end; r += kWaves) mx = fmaxf(mx, fabsf(v[(bh * m.L + r) * m.d + c]));
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
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t key = (int64_t)kc * 64 + 16 * q4 + i;
      const float x = c < m.d ? v[(bh * m.L + key) * m.d + c] : 0.0f;
      w[i / 4] |= ((uint32_t)code_w(x, s) & 0xFFu) << (8 * (i % 4));
    }
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
};

// Kept-block range of a query block, clamped to [0, nnz].
__device__ __forceinline__ void block_range(const int32_t* row_ptr, int64_t r, int32_t nnz, int& j0, int& j1) {
  j0 = min(max(row_ptr[r], 0), nnz);
  j1 = min(max(row_ptr[r + 1], j0), nnz);
}

// Logits z of one kept key block for the wave's 32 rows: z[ct][r] at row
// 8·(r/4) + 4·(lane/32) + r%4 of the tile and key 32·ct + lane%32 of the block.
__device__ __forceinline__ void block_logits(const ScoreArgs& a, int64_t bh, int kb, const v4i (&A)[kMaxKs][kPlanes],
                                             int np, int nks, float (&z)[2][16]) {
  const int lane = threadIdx.x & 63, li = lane & 31, hi = lane >> 5;
  const int8_t* kbase = a.kc + (bh * a.m.L + (int64_t)kb * kBlock) * a.m.dp;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    v4i Bf[kMaxKs];
#pragma unroll
    for (int ks = 0; ks < kMaxKs; ++ks)
      if (ks < nks) Bf[ks] = *reinterpret_cast<const v4i*>(kbase + (int64_t)(32 * ct + li) * a.m.dp + 32 * ks + 16 * hi);
    const double f = (double)a.ks[bh * a.m.L + (int64_t)kb * kBlock + 32 * ct + li] * a.g;
    int64_t s[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0;
#pragma unroll
    for (int jp = 0; jp < kPlanes; ++jp) {
      if (jp < np) {
        v16i acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0;
#pragma unroll
        for (int ks = 0; ks < kMaxKs; ++ks)
          if (ks < nks) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[ks][jp], Bf[ks], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] += (int64_t)acc[r] * ((int64_t)1 << (8 * jp));
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) z[ct][r] = (float)((double)s[r] * f);
  }
}

__global__ __launch_bounds__(kThreads) void scores_kernel(ScoreArgs a) {
  const int lane = threadIdx.x & 63, li = lane & 31, hi = lane >> 5;
  const int tpb = a.m.L / kTile;
  const int64_t tile = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (tile >= a.m.BH * tpb) return;
  const int64_t bh = tile / tpb;
  const int tau = (int)(tile % tpb);
  const int b = (int)(bh / a.m.heads), h = (int)(bh % a.m.heads);
  const int qb = tau >> 1, half = tau & 1;
  int j0, j1;
  block_range(a.row_ptr, (int64_t)h * a.m.nb + qb, a.nnz, j0, j1);
  if (j0 >= j1) return;
  const int nks = a.m.dp / 32;

  // Digit planes of a_Q for the tile (A operand, kept in registers).
  v4i A[kMaxKs][kPlanes];
  int pmax = 0;
  {
    const int8_t* qrow = a.qc + (bh * a.m.L + (int64_t)tau * kTile + li) * a.m.dp;
    const uint8_t* prow = a.qpot + (bh * tpb + tau) * a.m.dp;
#pragma unroll
    for (int ks = 0; ks < kMaxKs; ++ks) {
      if (ks < nks) {
        const v4i cw = *reinterpret_cast<const v4i*>(qrow + 32 * ks + 16 * hi);
        const v4i pw = *reinterpret_cast<const v4i*>(prow + 32 * ks + 16 * hi);
        pmax = max(pmax, digits16(cw, pw, A[ks]));
      } else {
#pragma unroll
        for (int j = 0; j < kPlanes; ++j) A[ks][j] = v4i{0, 0, 0, 0};
      }
    }
  }
  const int np = planes_for(wave_max_i(pmax));

  // Sweep 1: row maxima of the logits over every kept key.
  float mrow[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) mrow[r] = -INFINITY;
  for (int j = j0; j < j1; ++j) {
    const int kb = a.cols[j];
    if (kb < 0 || kb >= a.m.nb) continue;
    float z[2][16];
    block_logits(a, bh, kb, A, np, nks, z);
#pragma unroll
    for (int r = 0; r < 16; ++r) mrow[r] = fmaxf(mrow[r], fmaxf(z[0][r], z[1][r]));
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) mrow[r] = half_max(mrow[r]);

  // Sweep 2: exact sums of the fixed-point exponentials.
  int64_t srow[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) srow[r] = 0;
  for (int j = j0; j < j1; ++j) {
    const int kb = a.cols[j];
    if (kb < 0 || kb >= a.m.nb) continue;
    float z[2][16];
    block_logits(a, bh, kb, A, np, nks, z);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      srow[r] += exp_fixed(__fsub_rn(z[0][r], mrow[r])) + exp_fixed(__fsub_rn(z[1][r], mrow[r]));
  }
  double inv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) inv[r] = 1.0 / (double)half_sum(srow[r]);

  // Sweep 3: P, its FMDQ-INT8 codes per (tile, key) sub-channel, the cache.
  for (int j = j0; j < j1; ++j) {
    const int kb = a.cols[j];
    if (kb < 0 || kb >= a.m.nb) continue;
    float z[2][16];
    block_logits(a, bh, kb, A, np, nks, z);
    const int64_t blk = (int64_t)b * a.nnz + j;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float P[16];
      float mx = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        P[r] = (float)((double)exp_fixed(__fsub_rn(z[ct][r], mrow[r])) * inv[r]);
        mx = fmaxf(mx, P[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));    // the other 16 rows of the column
      const int pot = pot_of(mx, a.base_p);
      int8_t* dst = a.pc + (blk * kBlock + 32 * half) * kBlock + 32 * ct + li;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dst[(8 * (r >> 2) + 4 * hi + (r & 3)) * kBlock] = (int8_t)code8(P[r], a.inv_base_p, pot);
      if (hi == 0) a.ppot[(blk * 2 + half) * kBlock + 32 * ct + li] = (uint8_t)pot;
    }
  }
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

__global__ __launch_bounds__(kThreads) void pv_kernel(PvArgs a) {
  const int lane = threadIdx.x & 63, li = lane & 31, hi = lane >> 5;
  const int tpb = a.m.L / kTile;
  const int64_t tile = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (tile >= a.m.BH * tpb) return;
  const int64_t bh = tile / tpb;
  const int tau = (int)(tile % tpb);
  const int b = (int)(bh / a.m.heads), h = (int)(bh % a.m.heads);
  const int qb = tau >> 1, half = tau & 1;
  const int nct = a.m.dp / 32;
  int j0, j1;
  block_range(a.row_ptr, (int64_t)h * a.m.nb + qb, a.nnz, j0, j1);

  int64_t o[kMaxKs][16];
#pragma unroll
  for (int ct = 0; ct < kMaxKs; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[ct][r] = 0;

  for (int j = j0; j < j1; ++j) {
    const int kb = a.cols[j];
    if (kb < 0 || kb >= a.m.nb) continue;
    const int64_t blk = (int64_t)b * a.nnz + j;
    const int8_t* prow = a.pc + (blk * kBlock + 32 * half + li) * kBlock;
    const uint8_t* pp = a.ppot + (blk * 2 + half) * kBlock;
    v4i A[2][kPlanes];
    int pmax = 0;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const v4i cw = *reinterpret_cast<const v4i*>(prow + 32 * ks + 16 * hi);
      const v4i pw = *reinterpret_cast<const v4i*>(pp + 32 * ks + 16 * hi);
      pmax = max(pmax, digits16(cw, pw, A[ks]));
    }
    const int np = planes_for(wave_max_i(pmax));
#pragma unroll
    for (int ct = 0; ct < kMaxKs; ++ct) {
      if (ct < nct) {
        const int8_t* vrow = a.vct + (bh * a.m.dp + 32 * ct + li) * a.m.L + (int64_t)kb * kBlock + 16 * hi;
        const v4i B0 = *reinterpret_cast<const v4i*>(vrow);
        const v4i B1 = *reinterpret_cast<const v4i*>(vrow + 32);
#pragma unroll
        for (int jp = 0; jp < kPlanes; ++jp) {
          if (jp < np) {
            v16i acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0;
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[0][jp], B0, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[1][jp], B1, acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) o[ct][r] += (int64_t)acc[r] * ((int64_t)1 << (8 * jp));
          }
        }
      }
    }
  }

#pragma unroll
  for (int ct = 0; ct < kMaxKs; ++ct) {
    const int c = 32 * ct + li;
    if (ct < nct && c < a.m.d) {
      const double hc = (double)a.vscale[bh * a.m.d + c] * a.hp;
      float* dst = a.out + (bh * a.m.L + (int64_t)tau * kTile) * a.m.d + c;
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(int64_t)(8 * (r >> 2) + 4 * hi + (r & 3)) * a.m.d] = (float)((double)o[ct][r] * hc);
    }
  }
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
  hipLaunchKernelGGL(kquant_kernel, dim3(waves_grid(m.BH * m.L)), dim3(kThreads), 0, (hipStream_t)stream, k, kcodes,
                     kscale, m);
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
  if (nnz == 0) return DSTAR_OK;
  hipLaunchKernelGGL(scores_kernel, dim3(waves_grid(a.m.BH * (a.m.L / kTile))), dim3(kThreads), 0,
                     (hipStream_t)stream, a);
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
  hipLaunchKernelGGL(pv_kernel, dim3(waves_grid(a.m.BH * (a.m.L / kTile))), dim3(kThreads), 0, (hipStream_t)stream, a);
  return check_launch("sar_pv");
}

}  // extern "C"
