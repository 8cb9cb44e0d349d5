// Stage 3 of the FMDQ differential linear, MFMA kernel for gfx950 (DSTAR, arXiv
// 2607.15846: §3.1 steps 3 and 5 with Fig. 6; §4.2 MPU with its inverse
// quantization and accumulation units; §4.3 reverse differential fused into
// the GEMM).
//
// What is computed.  For an output (row t of token tile τ, column n)
//     S = Σ_k q[t][k] · 2^e_k · W[k][n]              (e_k = 15 − tag_k)
//     Y_t = fl32(f64(Y_{t−1}) + (f64(S) · f64(base)) · f64(w_scale[n]))
// which is the sum of the FPoT-group partial sums aligned by left shifts
// (§3.1 step 5: Σ_g acc_g · 2^(15−g)), dequantized and added to the cached
// output.  S is an exact integer; this kernel computes it exactly, so Y_t is
// the same float as the per-group formulation gives.
//
// How.  A sub-channel's code q (|q| ≤ 2^p, p = b − 2) at step 2^e has the
// value q·2^e in units of the base, and |q·2^e| ≤ 2^PoT.  When PoT ≤ 6 that
// shifted code still fits in int8: these sub-channels are "aligned" by the
// left shift of §3.1 step 5 before the multiply instead of after it, and all
// of them are summed by one natural-order int8 MFMA GEMM whose W chunks are
// staged once in LDS and shared by every token tile of the workgroup.  The few
// sub-channels with PoT ≥ 7 (only 8-bit ones at the default threshold) keep
// their own FPoT groups: each tile's such channels are gathered, grouped by
// tag in ascending FPoT, and multiplied group after group into the same int32
// accumulator, which is shifted left by the FPoT difference at every group
// change and finally to units of the base — the Horner form of the shift
// alignment of §3.1 step 5 and Fig. 6.  The dense GEMM then accumulates on
// top.
//
// Exactness.  int32 arithmetic wraps modulo 2^32, so the final accumulator
// equals S whenever |S| < 2^31; |S| ≤ 127 · Σ_k 2^PoT_k, so a token tile is
// handled here only if 127 · Σ_k 2^PoT_k < 2^31 and its gathered channel list
// fits the LDS budget.  Any other tile ("ineligible") is finished by an exact
// scalar path in the same workgroup that walks the tile's FPoT-ordered channel
// list (perm, group_off from stage 2) group by group with int32 group sums
// shifted into an int64 sum.
//
// Layout.  Workgroup = 256 threads = 4 waves, output block 128 rows × 128
// columns, 2 × 2 waves of 64 × 64 (2 × 2 MFMA 32x32x32 int8 tiles each).
// Codes ([tile][K][T], channel-major) and W ([K][N], row-major) both have the
// reduction index outermost, and so do their LDS copies: a chunk of 64
// channels is copied with 16-byte coalesced loads into [channel][row] and
// [channel][column] tiles (the code shift of a channel is one shift of each
// 16-byte piece).  Each lane then assembles its 16-byte MFMA fragment (one
// row or column, 16 consecutive channels) with two ds_read_b64_tr_b8
// transpose reads.  Chunks are double-buffered in LDS with one barrier per
// chunk, and the next chunk's global loads are in flight during the MFMAs.
#include "fmdq_internal.h"

namespace dstar {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int kThreads = 256;
constexpr int BM = 128;            // rows per workgroup
constexpr int BN = 128;            // output columns per workgroup
constexpr int BK = 64;             // channels per dense chunk (2 MFMA k-steps)
constexpr int KS = 32;             // channels per MFMA k-step
constexpr int SA = BM + 32;        // LDS bytes per channel row of an A tile
constexpr int SB = BN + 32;        // LDS bytes per channel row of a B tile
constexpr int kTags = DSTAR_FMDQ_NUM_TAGS;
constexpr int kAlignedPotMax = 6;  // q·2^e fits int8 when PoT ≤ 6
constexpr uint64_t kBoundLimit = 2147483647ull / 127ull;  // Σ 2^PoT limit
constexpr int kListBytes = 32768;  // gathered channel lists per workgroup
constexpr uint16_t kPad = 0xFFFFu;

template <int T>
struct Cfg {
  static constexpr int kTiles = BM / T;                   // token tiles per workgroup
  static constexpr int kCap = kListBytes / 2 / kTiles;    // list entries per tile
  static constexpr int kMaxSteps = kCap / KS;             // gathered k-steps per tile
};

// LDS carve-up (bytes): two A and two B chunk buffers, then the lists.
constexpr int kSizeA = BK * SA;                            // 10240
constexpr int kSizeB = BK * SB;                            // 10240
constexpr int kOffA0 = 0;
constexpr int kOffA1 = kOffA0 + kSizeA;
constexpr int kOffB0 = kOffA1 + kSizeA;
constexpr int kOffB1 = kOffB0 + kSizeB;
constexpr int kOffList = kOffB1 + kSizeB;                  // uint16 lists
constexpr int kOffStep = kOffList + kListBytes;            // uint8 step exponents
constexpr int kSizeStep = 4 * 128;
constexpr int kOffCnt = kOffStep + kSizeStep;              // uint32 [4][16] counters
constexpr int kOffCur = kOffCnt + 4 * kTags * 4;           // uint32 [4][16] cursors
constexpr int kOffBnd = kOffCur + 4 * kTags * 4;           // uint64 [4] bounds
constexpr int kOffMeta = kOffBnd + 4 * 8;                  // int32 [4] steps, [4] eligible
constexpr int kLdsBytes = kOffMeta + 8 * 4;
static_assert(Cfg<32>::kMaxSteps * 4 <= kSizeStep && Cfg<64>::kMaxSteps * 2 <= kSizeStep, "steps");
// Gathered steps keep A in buffer A0 (32 channel rows) and one B tile per
// token tile (32 channel rows of SB bytes each) in B0..B1.
static_assert(4 * KS * SB <= 2 * kSizeB, "gathered B tiles must fit");

// Left shift of four packed int8 codes by e (0..6); each result fits int8.
__device__ __forceinline__ uint32_t shift_codes(uint32_t x, int e) {
  const uint32_t m = 0x01010101u * ((0xFFu << e) & 0xFFu);
  return (x << e) & m;
}

// Decodes a tag byte: step exponent e = 15 − tag, PoT = e + (b − 2).
__device__ __forceinline__ int tag_e(uint32_t byte) { return DSTAR_FMDQ_TAG_OFFSET - (int)(byte & 15u); }
__device__ __forceinline__ int tag_pot(uint32_t byte) {
  return tag_e(byte) + 2 * (int)((byte >> DSTAR_FMDQ_PREC_SHIFT) & 3u);
}

__device__ __forceinline__ uint32_t ld_u32(const void* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}
__device__ __forceinline__ uint4 ld_u128(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st_u128(uint8_t* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// MFMA fragment from a [channel][row] LDS tile with row stride S: the lane
// gets row/column (lane % 32) and channels k0 + 16·(lane / 32) + 0..15.  Two
// transpose reads; in each 16-lane group, lane r addresses channel row
// k + r/2 at column offset 8·(r % 2) (+16 for the odd groups).
template <int S>
__device__ __forceinline__ v4i tr_frag(const uint8_t* tile, int k0, int col0, int lane) {
  const int q = lane >> 4, r = lane & 15;
  const uint8_t* p = tile + (k0 + 16 * (q >> 1) + (r >> 1)) * S + col0 + 16 * (q & 1) + 8 * (r & 1);
  const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)p);
  const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p + 8 * S));
  return v4i{lo[0], lo[1], hi[0], hi[1]};
}

__device__ __forceinline__ void shift_acc(v16i& acc, int s) {
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = (int)((uint32_t)acc[r] << s);
}

template <int T>
__global__ __launch_bounds__(kThreads, 2) void linear_mfma_kernel(LinearArgs a, int32_t col_blocks,
                                                                  int32_t vec_w) {
  using C = Cfg<T>;
  extern __shared__ __align__(16) uint8_t smem[];
  auto Abuf = [&](int b) { return smem + kOffA0 + b * kSizeA; };
  auto Bbuf = [&](int b) { return smem + kOffB0 + b * kSizeB; };
  uint16_t* list = reinterpret_cast<uint16_t*>(smem + kOffList);       // [kTiles][kCap]
  uint8_t* step_e = smem + kOffStep;                                    // [kTiles][kMaxSteps]
  uint32_t* cnt = reinterpret_cast<uint32_t*>(smem + kOffCnt);         // [kTiles][16]
  uint32_t* cur = reinterpret_cast<uint32_t*>(smem + kOffCur);         // [kTiles][16]
  unsigned long long* bnd = reinterpret_cast<unsigned long long*>(smem + kOffBnd);
  int32_t* nsteps = reinterpret_cast<int32_t*>(smem + kOffMeta);       // [4]
  int32_t* eligible = nsteps + 4;                                       // [4]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t K = a.K, N = a.N;
  const int64_t nt = n_tiles(a.rows, T);
  const int64_t mb = blockIdx.x / col_blocks;
  const int64_t n0 = (int64_t)(blockIdx.x - mb * col_blocks) * BN;
  const int64_t tile0 = mb * C::kTiles;
  const int tiles_here = (int)min<int64_t>(C::kTiles, nt - tile0);

  // ---- Prologue: per tile, the channels whose aligned codes exceed int8,
  // grouped by tag in ascending FPoT, each group padded to a whole k-step.
  if (tid < C::kTiles * kTags) cnt[tid] = 0u;
  if (tid < C::kTiles) bnd[tid] = 0ull;
  __syncthreads();
  const int64_t kq_total = (K / 4) * tiles_here;   // tag words of this block's tiles
  {
    unsigned long long b[C::kTiles];
#pragma unroll
    for (int i = 0; i < C::kTiles; ++i) b[i] = 0;
    for (int64_t base = tid; base < kq_total; base += 4 * kThreads) {
      uint32_t w[4];
      int64_t idx[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        idx[u] = base + u * kThreads;
        w[u] = idx[u] < kq_total ? ld_u32(a.tags + tile0 * K + 4 * idx[u]) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (idx[u] >= kq_total) continue;
        const int i = (int)(idx[u] / (K / 4));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t byte = (w[u] >> (8 * c)) & 0xFFu;
          const int pot = tag_pot(byte);
#pragma unroll
          for (int ii = 0; ii < C::kTiles; ++ii)
            if (ii == i) b[ii] += 1ull << pot;
          if (pot > kAlignedPotMax) atomicAdd(&cnt[i * kTags + (byte & 15u)], 1u);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::kTiles; ++i) {
      unsigned long long v = b[i];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
      if (lane == 0 && i < tiles_here) atomicAdd(&bnd[i], v);
    }
  }
  __syncthreads();
  if (tid < C::kTiles) {
    const int i = tid;
    int total = 0;
    for (int g = 0; g < kTags; ++g) {
      cur[i * kTags + g] = (uint32_t)total;
      total += (int)((cnt[i * kTags + g] + KS - 1) / KS) * KS;
    }
    const bool ok = i < tiles_here && total <= C::kCap && bnd[i] <= kBoundLimit;
    eligible[i] = ok ? 1 : 0;
    nsteps[i] = ok ? total / KS : 0;
    if (ok) {
      for (int g = 0; g < kTags; ++g) {
        const int s0 = (int)cur[i * kTags + g] / KS;
        const int ns = (int)((cnt[i * kTags + g] + KS - 1) / KS);
        for (int s = s0; s < s0 + ns; ++s) step_e[i * C::kMaxSteps + s] = (uint8_t)(DSTAR_FMDQ_TAG_OFFSET - g);
      }
    }
  }
  __syncthreads();
  for (int i = 0; i < C::kTiles; ++i) {
    const int len = nsteps[i] * KS;
    for (int j = tid; j < len; j += kThreads) list[i * C::kCap + j] = kPad;
  }
  __syncthreads();
  for (int64_t base = tid; base < kq_total; base += 4 * kThreads) {
    uint32_t w[4];
    int64_t idx[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      idx[u] = base + u * kThreads;
      const int i = idx[u] < kq_total ? (int)(idx[u] / (K / 4)) : 0;
      w[u] = (idx[u] < kq_total && nsteps[i] > 0) ? ld_u32(a.tags + tile0 * K + 4 * idx[u]) : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (idx[u] >= kq_total) continue;
      const int i = (int)(idx[u] / (K / 4));
      if (nsteps[i] == 0) continue;
      const int64_t k = 4 * (idx[u] - (int64_t)i * (K / 4));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t byte = (w[u] >> (8 * c)) & 0xFFu;
        if (tag_pot(byte) > kAlignedPotMax) {
          const uint32_t slot = atomicAdd(&cur[i * kTags + (byte & 15u)], 1u);
          list[i * C::kCap + slot] = (uint16_t)(k + c);
        }
      }
    }
  }
  __syncthreads();

  v16i acc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0;

  // Tile of each of this wave's two 32-row MFMA blocks.
  int rb_tile[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) rb_tile[rb] = (64 * wr + 32 * rb) / T;

  // ---- Gathered FPoT groups, Horner form: ascending tag = descending step.
  int max_steps = 0;
#pragma unroll
  for (int i = 0; i < C::kTiles; ++i) max_steps = max(max_steps, nsteps[i]);
  for (int s = 0; s < max_steps; ++s) {
    __syncthreads();
    // A: per tile, 32 gathered channels × T rows -> Abuf(0)[entry][T·i + t].
    {
      constexpr int kPieces = T / 16;                  // 16-byte pieces per channel
      const int p = tid;                               // kTiles · 32 · kPieces = 256
      const int i = p / (KS * kPieces);
      const int j = (p / kPieces) % KS;
      const int sub = p % kPieces;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (s < nsteps[i]) {
        const uint16_t ch = list[i * C::kCap + s * KS + j];
        if (ch != kPad) v = ld_u128(a.codes + ((tile0 + i) * K + ch) * T + 16 * sub);
      }
      st_u128(Abuf(0) + j * SA + T * i + 16 * sub, v);
    }
    // B: per tile, 32 gathered W rows × 128 columns -> [entry][column].
#pragma unroll
    for (int i = 0; i < C::kTiles; ++i) {
      if (s >= nsteps[i]) continue;
      const int j = tid >> 3, c16 = tid & 7;           // 32 rows × 8 pieces
      const uint16_t ch = list[i * C::kCap + s * KS + j];
      const int64_t n = n0 + 16 * c16;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (ch != kPad) {
        const int8_t* src = a.w + (int64_t)ch * N + n;
        if (vec_w && n + 16 <= N) {
          v = ld_u128(src);
        } else {
          uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int m = 0; m < 4; ++m)
            if (n + 4 * m < N) d[m] = ld_u32(src + 4 * m);
          v = make_uint4(d[0], d[1], d[2], d[3]);
        }
      }
      st_u128(smem + kOffB0 + i * KS * SB + j * SB + 16 * c16, v);
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int i = rb_tile[rb];
      if (s >= nsteps[i]) continue;
      const int e = step_e[i * C::kMaxSteps + s];
      if (s > 0) {
        const int ep = step_e[i * C::kMaxSteps + s - 1];
        if (ep != e) {
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) shift_acc(acc[rb][cb], ep - e);
        }
      }
      const v4i af = tr_frag<SA>(Abuf(0), 0, 64 * wr + 32 * rb, lane);
      const uint8_t* Bt = smem + kOffB0 + i * KS * SB;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const v4i bf = tr_frag<SB>(Bt, 0, 64 * wc + 32 * cb, lane);
        acc[rb][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf, acc[rb][cb], 0, 0, 0);
      }
    }
  }
  // Bring the gathered groups to units of the base (step 2^0).
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int i = rb_tile[rb];
    if (nsteps[i] > 0) {
      const int e = step_e[i * C::kMaxSteps + nsteps[i] - 1];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) shift_acc(acc[rb][cb], e);
    }
  }

  // ---- Dense part: every other channel, natural order, codes shifted by e.
  // A chunk: per tile, 64 channels × T rows (contiguous in memory) as 16-byte
  // pieces; B chunk: 64 W rows × 128 columns as 16-byte pieces.
  constexpr int kPiecesA = BK * BM / 16 / kThreads;    // 2
  constexpr int kPiecesB = BK * BN / 16 / kThreads;    // 2
  uint4 ra[kPiecesA], rbv[kPiecesB];
  uint32_t rtag[kPiecesA];
  auto load_chunk = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < kPiecesA; ++u) {
      const int p = tid + kThreads * u;
      const int i = p / (BK * T / 16);
      const int q = p % (BK * T / 16);
      const int kk = q / (T / 16);
      ra[u] = make_uint4(0u, 0u, 0u, 0u);
      rtag[u] = 0xFFu;  // decodes to PoT > 6: contributes nothing
      if (i < tiles_here && k0 + kk < K) {
        ra[u] = ld_u128(a.codes + ((tile0 + i) * K + k0) * T + 16 * q);
        rtag[u] = a.tags[(tile0 + i) * K + k0 + kk];
      }
    }
#pragma unroll
    for (int u = 0; u < kPiecesB; ++u) {
      const int p = tid + kThreads * u;
      const int kk = p / (BN / 16), c16 = p % (BN / 16);
      const int64_t n = n0 + 16 * c16;
      rbv[u] = make_uint4(0u, 0u, 0u, 0u);
      if (k0 + kk < K) {
        const int8_t* src = a.w + (k0 + kk) * N + n;
        if (vec_w && n + 16 <= N) {
          rbv[u] = ld_u128(src);
        } else {
          uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int m = 0; m < 4; ++m)
            if (n + 4 * m < N) d[m] = ld_u32(src + 4 * m);
          rbv[u] = make_uint4(d[0], d[1], d[2], d[3]);
        }
      }
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kPiecesA; ++u) {
      const int p = tid + kThreads * u;
      const int i = p / (BK * T / 16);
      const int q = p % (BK * T / 16);
      const int kk = q / (T / 16), sub = q % (T / 16);
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (tag_pot(rtag[u]) <= kAlignedPotMax) {
        const int e = tag_e(rtag[u]);
        v = make_uint4(shift_codes(ra[u].x, e), shift_codes(ra[u].y, e), shift_codes(ra[u].z, e),
                       shift_codes(ra[u].w, e));
      }
      st_u128(Abuf(buf) + kk * SA + T * i + 16 * sub, v);
    }
#pragma unroll
    for (int u = 0; u < kPiecesB; ++u) {
      const int p = tid + kThreads * u;
      const int kk = p / (BN / 16), c16 = p % (BN / 16);
      st_u128(Bbuf(buf) + kk * SB + 16 * c16, rbv[u]);
    }
  };

  const int64_t nchunks = (K + BK - 1) / BK;
  __syncthreads();  // the gathered steps are done with the buffers
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int64_t c = 0; c < nchunks; ++c) {
    const int buf = (int)(c & 1);
    if (c + 1 < nchunks) load_chunk((c + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / KS; ++ks) {
      v4i af[2], bf[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) af[rb] = tr_frag<SA>(Abuf(buf), KS * ks, 64 * wr + 32 * rb, lane);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) bf[cb] = tr_frag<SB>(Bbuf(buf), KS * ks, 64 * wc + 32 * cb, lane);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[rb], bf[cb], acc[rb][cb], 0, 0, 0);
    }
    if (c + 1 < nchunks) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // ---- Epilogue: dequantize, add the cached output, store (float64 combine).
  // Y is streamed once, so it bypasses the caches that hold W and the codes;
  // every load of the cached output is issued before the first store.
  const double base = a.base;
  const int h = lane >> 5, li = lane & 31;
  bool all_eligible = true;
#pragma unroll
  for (int i = 0; i < C::kTiles; ++i) all_eligible = all_eligible && eligible[i];
  const bool interior = all_eligible && (tile0 * T + BM <= a.rows) && (n0 + BN <= N);
  if (interior) {
    float yp[2][2][16];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = tile0 * T + 64 * wr + 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
          yp[rb][cb][r] = __builtin_nontemporal_load(a.y_prev + row * N + n0 + 64 * wc + 32 * cb + li);
        }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int64_t n = n0 + 64 * wc + 32 * cb + li;
      const double ws = (double)a.w_scale[n];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = tile0 * T + 64 * wr + 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
          const double d = __dmul_rn(__dmul_rn((double)acc[rb][cb][r], base), ws);
          __builtin_nontemporal_store((float)__dadd_rn((double)yp[rb][cb][r], d), a.y_out + row * N + n);
        }
    }
  } else {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int64_t n = n0 + 64 * wc + 32 * cb + li;
      if (n >= N) continue;
      const double ws = (double)a.w_scale[n];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int i = rb_tile[rb];
        if (!eligible[i]) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 64 * wr + 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
          const int64_t grow = tile0 * T + row;
          if (grow >= a.rows) continue;
          const int64_t idx = grow * N + n;
          const double d = __dmul_rn(__dmul_rn((double)acc[rb][cb][r], base), ws);
          a.y_out[idx] = (float)__dadd_rn((double)a.y_prev[idx], d);
        }
      }
    }
  }

  // ---- Ineligible tiles: exact scalar path over the FPoT-ordered channels
  // (stage 2's perm and group offsets), int32 group sums shifted into int64.
  for (int i = 0; i < tiles_here; ++i) {
    if (eligible[i]) continue;
    const int64_t tau = tile0 + i;
    constexpr int kRowSets = kThreads / BN;           // 2
    constexpr int kRows = T / kRowSets;               // rows per thread
    const int64_t n = n0 + (tid % BN);
    const int t0 = (tid / BN) * kRows;
    if (n >= N) continue;
    const int32_t* off = a.group_off + tau * (kTags + 1);
    const uint16_t* pm = a.perm + tau * K;
    const int8_t* cd = a.codes + tau * K * T;
    int64_t sum[kRows];
#pragma unroll
    for (int t = 0; t < kRows; ++t) sum[t] = 0;
    for (int g = 0; g < kTags; ++g) {
      const int lo = off[g], hi = off[g + 1];
      if (lo == hi) continue;
      int32_t gs[kRows];
#pragma unroll
      for (int t = 0; t < kRows; ++t) gs[t] = 0;
      for (int j = lo; j < hi; ++j) {
        const int64_t k = pm[j];
        const int32_t wv = (int32_t)a.w[k * N + n];
        const int4* c4 = reinterpret_cast<const int4*>(cd + k * T + t0);
#pragma unroll
        for (int v = 0; v < kRows / 16; ++v) {
          const int4 c = c4[v];
          const int words[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
          for (int b = 0; b < 16; ++b) gs[16 * v + b] += (int32_t)(int8_t)(words[b >> 2] >> (8 * (b & 3))) * wv;
        }
      }
#pragma unroll
      for (int t = 0; t < kRows; ++t) sum[t] += (int64_t)gs[t] << (DSTAR_FMDQ_TAG_OFFSET - g);
    }
    const double ws = (double)a.w_scale[n];
#pragma unroll
    for (int t = 0; t < kRows; ++t) {
      const int64_t grow = tau * T + t0 + t;
      if (grow >= a.rows) continue;
      const int64_t idx = grow * N + n;
      const double d = __dmul_rn(__dmul_rn((double)sum[t], base), ws);
      a.y_out[idx] = (float)__dadd_rn((double)a.y_prev[idx], d);
    }
  }
}

template <int T>
int launch_t(const LinearArgs& a, hipStream_t s) {
  const int64_t nt = n_tiles(a.rows, T);
  const int64_t row_blocks = (nt + Cfg<T>::kTiles - 1) / Cfg<T>::kTiles;
  const int32_t col_blocks = (int32_t)((a.N + BN - 1) / BN);
  const int64_t grid = row_blocks * col_blocks;
  if (grid > 0x7FFFFFFF) return set_error(DSTAR_EUNSUPPORTED, "fmdq_linear: grid too large");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)linear_mfma_kernel<T>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess)
      return set_error(DSTAR_EHIP, "fmdq_linear: hipFuncSetAttribute: %s", hipGetErrorString(e));
    attr_set = true;
  }
  const int32_t vec_w = (a.N % 16) == 0 ? 1 : 0;
  hipLaunchKernelGGL(linear_mfma_kernel<T>, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, s, a,
                     col_blocks, vec_w);
  return check_launch("fmdq_linear (mfma)");
}

}  // namespace

// Handles token tiles of 32 or 64 rows with K a multiple of 4.
bool linear_mfma_supported(const LinearArgs& a) {
  return (a.T == 32 || a.T == 64) && (a.K % 4) == 0;
}

int launch_linear_mfma(const LinearArgs& a, hipStream_t s) {
  switch (a.T) {
    case 32: return launch_t<32>(a, s);
    case 64: return launch_t<64>(a, s);
    default: return set_error(DSTAR_EUNSUPPORTED, "fmdq_linear (mfma): token_tile %d", a.T);
  }
}

}  // namespace dstar
