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
// handled here only if 127 · Σ_k 2^PoT_k < 2^31 (computed from stage 2's bin
// counts).  Any other tile ("ineligible") is finished by an exact scalar path
// in the same workgroup that walks the tile's FPoT groups in perm order with
// int32 group sums shifted into an int64 sum.
//
// Stage 2 orders each FPoT group widest precision first, so the channels of a
// group with PoT ≥ 7 are a prefix of the group in perm, found from the bin
// offsets alone; the gathered steps read perm directly.
//
// Layout.  Workgroup = 256 threads = 4 waves, output block 128 rows × 256
// columns; wave w owns all 128 rows and columns 64w .. 64w+63 (4 × 2 MFMA
// 32x32x32 int8 tiles).  Dense part: 64-channel chunks of stage 1's aligned
// codes ([rows][K]) and of W^T ([N][K]), both channel innermost, flow through
// a 3-stage LDS ring filled by direct global-to-LDS buffer loads, two chunks
// ahead of the MFMAs; the four 16-byte columns of every 64-byte row are
// XOR-swizzled by (row / 4) mod 4 so that one ds_read_b128 per fragment is
// free of bank conflicts.  The aligned-code rows are shared by the four waves,
// each wave reads only its own 64 W^T rows.  Gathered part: the codes
// ([tile][K][T]) and W ([K][N]) rows of the gathered channels have the channel
// outermost; they are staged as [channel][row] and [channel][column] LDS tiles
// and each lane assembles its fragment (one row or column, 16 consecutive
// channels) with two ds_read_b64_tr_b8 transpose reads; perm entries are
// fetched two steps and data one step ahead.
#include "fmdq_internal.h"

namespace dstar {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int BM = 128;            // rows per workgroup
constexpr int WN = 64;             // output columns per wave
constexpr int BN = kWaves * WN;    // output columns per workgroup (256)
constexpr int RB = BM / 32;        // 32-row MFMA blocks per wave (4)
constexpr int CB = WN / 32;        // 32-column MFMA blocks per wave (2)
constexpr int BK = 64;             // channels per dense chunk (2 MFMA k-steps)
constexpr int KS = 32;             // channels per MFMA k-step (= per gathered step)
constexpr int SA = BM + 32;        // LDS bytes per channel row of the gathered A tile
constexpr int SB = BN + 32;        // LDS bytes per channel row of a gathered B tile
constexpr int kTags = DSTAR_FMDQ_NUM_TAGS;
constexpr int kBins = DSTAR_FMDQ_NUM_BINS;
constexpr int kAlignedPotMax = 6;  // q·2^e fits int8 when PoT ≤ 6
constexpr uint64_t kBoundLimit = 2147483647ull / 127ull;  // Σ 2^PoT limit
constexpr int kBand = 8;           // row blocks per band of the block order

template <int T>
struct Cfg {
  static constexpr int kTiles = BM / T;   // token tiles per workgroup
};

// LDS carve-up (bytes).  Dense: kStages stages of (A 128 rows + B 256 rows)
// × 64 bytes.  Gathered: one stage of (A: 32 channel rows; B: one 32-row tile
// per token tile).  The two phases reuse the same bytes.
constexpr int kStages = 3;
constexpr int kStageDense = (BM + BN) * BK;                // 24576
constexpr int kDenseBytes = kStages * kStageDense;         // 73728
constexpr int kStageBytes = KS * SA + 4 * KS * SB;         // 41984
constexpr int kDataBytes = kDenseBytes > kStageBytes ? kDenseBytes : kStageBytes;
constexpr int kOffOff = kDataBytes;                         // int32 [4][65] bin offsets
constexpr int kOffRs = kOffOff + 4 * (kBins + 1) * 4;      // int32 [4][16] prefix starts
constexpr int kOffRc = kOffRs + 4 * kTags * 4;             // int32 [4][16] prefix lengths
constexpr int kOffBp = kOffRc + 4 * kTags * 4;             // uint64 [4][16] bound parts
constexpr int kOffSteps = kOffBp + 4 * kTags * 8;          // int32 [16] steps per group
constexpr int kOffCum = kOffSteps + kTags * 4;             // int32 [17] cumulative steps
constexpr int kOffElig = kOffCum + (kTags + 1) * 4;        // int32 [4]
constexpr int kLdsBytes = kOffElig + 4 * 4;

__device__ __forceinline__ void st_u128(uint8_t* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// Operand loads go through buffer resources: a load whose offset lies outside
// the resource's byte range returns zeros, so every load is unconditional
// (an invalid piece is given the offset kOob) and the compiler can count the
// loads still in flight instead of waiting for all of them.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void* lds_ptr;
constexpr uint32_t kOob = 0x80000000u;
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; the unused counters at their maximum): wait until no
// vector-memory load is in flight, or at most one dense chunk's six loads.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitVmChunk = 0x0F76;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ v4i bload16v(rsrc_t r, uint32_t off) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return v4i{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// 16 bytes of W at byte offset `off` of the W resource; with VecW the piece is
// one 16-byte load (N % 16 == 0, the piece lies wholly inside or outside W),
// otherwise four 4-byte loads, each dropped past column N.
template <bool VecW>
__device__ __forceinline__ uint4 load_w16(rsrc_t rw, uint32_t off, int64_t n, int64_t N, bool valid) {
  if constexpr (VecW) {
    return bload16(rw, valid ? off : kOob);
  } else {
    uint32_t d[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) d[m] = bload4(rw, (valid && n + 4 * m < N) ? off + 4 * m : kOob);
    return make_uint4(d[0], d[1], d[2], d[3]);
  }
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

template <int T, bool VecW>
__global__ __launch_bounds__(kThreads, 2) void linear_mfma_kernel(LinearArgs a, int32_t row_blocks,
                                                                  int32_t col_blocks) {
  constexpr int kTiles = Cfg<T>::kTiles;
  extern __shared__ __align__(16) uint8_t smem[];
  int32_t* off_s = reinterpret_cast<int32_t*>(smem + kOffOff);          // [kTiles][65]
  int32_t* rstart = reinterpret_cast<int32_t*>(smem + kOffRs);          // [kTiles][16]
  int32_t* rcount = reinterpret_cast<int32_t*>(smem + kOffRc);          // [kTiles][16]
  unsigned long long* bpart = reinterpret_cast<unsigned long long*>(smem + kOffBp);
  int32_t* steps_g = reinterpret_cast<int32_t*>(smem + kOffSteps);      // [16]
  int32_t* cum = reinterpret_cast<int32_t*>(smem + kOffCum);            // [17]
  int32_t* eligible = reinterpret_cast<int32_t*>(smem + kOffElig);      // [kTiles]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31, h = lane >> 5;
  const int64_t K = a.K, N = a.N;
  const int64_t nt = n_tiles(a.rows, T);

  // Block order.  Workgroups are dealt to the 8 XCDs round-robin (XCD =
  // blockIdx % 8), each with its own L2.  XCD x takes a contiguous range of a
  // banded order of the (row block, column block) grid: bands of kBand row
  // blocks, walked column block by column block, so the workgroups an XCD
  // runs at the same time share their code rows and W columns in its L2.
  int64_t mb, nb;
  {
    const int64_t G = (int64_t)row_blocks * col_blocks;
    const int64_t x = blockIdx.x % 8, j = blockIdx.x / 8;
    const int64_t L = x * (G / 8) + min<int64_t>(x, G % 8) + j;
    const int64_t band = L / ((int64_t)kBand * col_blocks);
    const int64_t Lb = L % ((int64_t)kBand * col_blocks);
    const int64_t hgt = min<int64_t>(kBand, row_blocks - band * kBand);
    mb = band * kBand + Lb % hgt;
    nb = Lb / hgt;
  }
  const int64_t n0 = nb * BN;
  const int64_t nw = n0 + WN * wave;      // this wave's first column
  const int64_t tile0 = mb * kTiles;
  const int tiles_here = (int)min<int64_t>(kTiles, nt - tile0);
  // This workgroup's tiles of codes, aligned codes and perm; all of W, W^T.
  const rsrc_t r_codes = make_rsrc(a.codes + tile0 * K * T, (uint32_t)(tiles_here * K * T));
  const rsrc_t r_perm = make_rsrc(a.perm + tile0 * K, (uint32_t)(tiles_here * K * 2));
  const rsrc_t r_ac = make_rsrc(a.acodes + tile0 * T * K, (uint32_t)(tiles_here * T * K));
  const rsrc_t r_w = make_rsrc(a.w, (uint32_t)(K * N));
  const rsrc_t r_wt = make_rsrc(a.w_t, (uint32_t)(N * K));

  // ---- Meta: per tile and FPoT group, the prefix of the group (in perm)
  // whose channels have PoT ≥ 7, and the exactness bound Σ_k 2^PoT_k.
  for (int idx = tid; idx < kTiles * (kBins + 1); idx += kThreads) {
    const int i = idx / (kBins + 1);
    off_s[idx] = i < tiles_here ? a.group_off[(tile0 + i) * (kBins + 1) + idx % (kBins + 1)] : 0;
  }
  __syncthreads();
  if (tid < kTiles * kTags) {
    const int i = tid / kTags, g = tid % kTags;
    const int e = DSTAR_FMDQ_TAG_OFFSET - g;
    const int32_t* o = off_s + i * (kBins + 1);
    // PoT = e + 2·pc ≥ 7  <=>  pc ≥ ceil((7 − e) / 2); bins of group g run
    // from precision code 3 (bin 4g) down to 0 (bin 4g + 3).
    const int pcmin = max(0, (kAlignedPotMax + 2 - e) / 2);
    rstart[tid] = o[4 * g];
    rcount[tid] = pcmin <= 3 ? o[4 * g + 4 - pcmin] - o[4 * g] : 0;
    unsigned long long b = 0;
#pragma unroll
    for (int pc = 0; pc < 4; ++pc)
      b += (unsigned long long)(o[4 * g + 4 - pc] - o[4 * g + 3 - pc]) << (e + 2 * pc);
    bpart[tid] = b;
  }
  __syncthreads();
  if (tid < kTiles) {
    unsigned long long b = 0;
    for (int g = 0; g < kTags; ++g) b += bpart[tid * kTags + g];
    eligible[tid] = (tid < tiles_here && b <= kBoundLimit) ? 1 : 0;
  }
  __syncthreads();
  if (tid < kTags) {
    int m = 0;
#pragma unroll
    for (int i = 0; i < kTiles; ++i)
      if (eligible[i]) m = max(m, (rcount[i * kTags + tid] + KS - 1) / KS);
    steps_g[tid] = m;
  }
  __syncthreads();
  if (tid == 0) {
    cum[0] = 0;
    for (int g = 0; g < kTags; ++g) cum[g + 1] = cum[g] + steps_g[g];
  }
  __syncthreads();
  const int nsteps = cum[kTags];

  v16i acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0;

  // ---- Gathered FPoT groups, Horner form: ascending tag = descending step.
  // Step f of the workgroup covers entries 32·s .. 32·s + 31 of group g's
  // prefix in every tile.  Thread roles: A piece (tile iA, entry jA, 16-byte
  // piece subA of the channel's T codes); B pieces (entry jB, columns
  // n0 + 16·cB .. +15 and n0 + 128 + 16·cB .. +15) of every tile.
  {
    constexpr int kPieces = T / 16;
    const int iA = tid / (KS * kPieces), jA = (tid / kPieces) % KS, subA = tid % kPieces;
    const int jB = tid >> 3, cB = tid & 7;
    auto step_group = [&](int f, int& g, int& s) {
      g = 0;
      while (cum[g + 1] <= f) ++g;
      s = f - cum[g];
    };
    // Entries: the channel id (low 16 bits) and a valid flag (bit 16).
    uint32_t eA, eB[kTiles];
    uint4 dA, dB[kTiles][2];
    auto entry = [&](int i, int g, int j) -> uint32_t {
      const int cnt = eligible[i] ? rcount[i * kTags + g] : 0;
      const bool valid = j < cnt;
      const uint32_t off = (uint32_t)(i * K + rstart[i * kTags + g] + j) * 2u;
      return (__builtin_amdgcn_raw_buffer_load_b16(r_perm, valid ? off : kOob, 0, 0) & 0xFFFFu) |
             (valid ? 0x10000u : 0u);
    };
    auto entries = [&](int f) {
      int g, s;
      step_group(f, g, s);
      eA = entry(iA, g, KS * s + jA);
#pragma unroll
      for (int i = 0; i < kTiles; ++i) eB[i] = entry(i, g, KS * s + jB);
    };
    auto data = [&]() {
      const uint32_t chA = eA & 0xFFFFu;
      dA = bload16(r_codes, (eA >> 16) ? (uint32_t)((iA * K + chA) * T + 16 * subA) : kOob);
#pragma unroll
      for (int i = 0; i < kTiles; ++i) {
        const uint32_t ch = eB[i] & 0xFFFFu;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int64_t n = n0 + 128 * u + 16 * cB;
          dB[i][u] = load_w16<VecW>(r_w, (uint32_t)(ch * N + n), n, N, (eB[i] >> 16) && n < N);
        }
      }
    };
    auto store = [&]() {
      st_u128(smem + jA * SA + T * iA + 16 * subA, dA);
#pragma unroll
      for (int i = 0; i < kTiles; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          st_u128(smem + KS * SA + i * KS * SB + jB * SB + 128 * u + 16 * cB, dB[i][u]);
    };
    int prev_e[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) prev_e[rb] = -1;
    if (nsteps > 0) {
      entries(0);
      data();
      if (nsteps > 1) entries(1);
      for (int f = 0; f < nsteps; ++f) {
        __syncthreads();                 // the previous step's fragments are read
        store();
        __syncthreads();
        if (f + 1 < nsteps) data();      // entries of step f+1 arrived one step ago
        if (f + 2 < nsteps) entries(f + 2);
        int g, s;
        step_group(f, g, s);
        const int e = DSTAR_FMDQ_TAG_OFFSET - g;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int i = (32 * rb) / T;
          const int cnt = eligible[i] ? rcount[i * kTags + g] : 0;
          if (KS * s >= cnt) continue;
          if (s == 0) {
            if (prev_e[rb] >= 0) {
#pragma unroll
              for (int cb = 0; cb < CB; ++cb) shift_acc(acc[rb][cb], prev_e[rb] - e);
            }
            prev_e[rb] = e;
          }
          const v4i af = tr_frag<SA>(smem, 0, 32 * rb, lane);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const v4i bf = tr_frag<SB>(smem + KS * SA + i * KS * SB, 0, WN * wave + 32 * cb, lane);
            acc[rb][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf, acc[rb][cb], 0, 0, 0);
          }
        }
      }
    }
    // Bring the gathered groups to units of the base (step 2^0).
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      if (prev_e[rb] > 0) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) shift_acc(acc[rb][cb], prev_e[rb]);
      }
  }

  // ---- Dense part: every channel with PoT ≤ 6, natural order, 64 channels
  // per chunk through a ring of kStages LDS stages filled by direct
  // global-to-LDS loads (no registers): A = the 128 rows of aligned codes,
  // shared by the four waves; B = each wave's 64 columns of W^T.  Both tiles
  // are [row][64 channels] with the 16-byte columns XOR-swizzled by row,
  // (column ^ (row / 4) % 4), so the fragment reads (one ds_read_b128) are
  // free of bank conflicts.  A direct load writes lane l's 16 bytes at
  // base + 16·l: one wave instruction fills 16 rows.
  {
    auto stageA = [&](int st) { return smem + st * kStageDense; };
    auto stageB = [&](int st, int w) { return smem + st * kStageDense + BM * BK + w * WN * BK; };
    const int r16 = lane >> 2;                       // row of this lane within a 16-row group
    const int c16 = (lane & 3) ^ ((r16 >> 2) & 3);   // global 16-byte column it loads
    // Each wave issues 2 A and 4 B instructions per chunk.
    auto issue = [&](int64_t c, int st) {
      const int64_t k0 = c * BK;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 16 * (2 * wave + j) + r16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r_ac, (lds_ptr)(stageA(st) + 1024 * (2 * wave + j)), 16,
                                                 (uint32_t)(row * K + k0 + 16 * c16), 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = nw + 16 * j + r16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r_wt, (lds_ptr)(stageB(st, wave) + 1024 * j), 16,
                                                 n < N ? (uint32_t)(n * K + k0 + 16 * c16) : kOob, 0, 0, 0);
      }
    };
    auto frag = [&](const uint8_t* tile, int row, int c) {
      return *reinterpret_cast<const v4i*>(tile + row * BK + 16 * (c ^ ((row >> 2) & 3)));
    };
    auto compute = [&](int st) {
#pragma unroll
      for (int ks = 0; ks < BK / KS; ++ks) {
        v4i af[RB], bf[CB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) af[rb] = frag(stageA(st), 32 * rb + li, 2 * ks + h);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) bf[cb] = frag(stageB(st, wave), 32 * cb + li, 2 * ks + h);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[rb], bf[cb], acc[rb][cb], 0, 0, 0);
      }
    };

    const int64_t nchunks = K / BK;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // no other vector loads in flight
    __syncthreads();                        // the gathered steps are done with LDS
#pragma unroll
    for (int c = 0; c < kStages - 1; ++c)
      if (c < nchunks) issue(c, c);
    for (int64_t c = 0; c < nchunks; ++c) {
      // Chunk c's loads are done once at most one later chunk is in flight.
      // A bare s_barrier then makes every wave's part of chunk c visible and
      // guarantees every wave is done with chunk c - 1 (whose stage the next
      // loads overwrite).  (__syncthreads would also wait for the loads still
      // in flight, which is what the stages are there to avoid.)  The empty
      // asm statements keep the compiler from moving LDS reads across.
      if (c + 1 < nchunks) {
        __builtin_amdgcn_s_waitcnt(kWaitVmChunk);
      } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      }
      __asm__ __volatile__("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ __volatile__("" ::: "memory");
      if (c + kStages - 1 < nchunks) issue(c + kStages - 1, (int)((c + kStages - 1) % kStages));
      compute((int)(c % kStages));
    }
  }

  // ---- Epilogue: dequantize, add the cached output, store (float64 combine).
  // Y is streamed once: its loads and stores are non-temporal so they do not
  // evict W and the codes from the caches.  In interior blocks the 32 loads
  // of one 32-row block of the wave are issued before their stores.  Offsets
  // are 32-bit, relative to this workgroup's first row.
  const double base = a.base;
  bool all_eligible = true;
#pragma unroll
  for (int i = 0; i < kTiles; ++i) all_eligible = all_eligible && eligible[i];
  const bool interior = all_eligible && (tile0 * T + BM <= a.rows) && (nw + WN <= N);
  double ws[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int64_t n = nw + 32 * cb + li;
    ws[cb] = n < N ? (double)a.w_scale[n] : 0.0;
  }
  if (interior) {
    constexpr int kNt = 2;   // aux bit: non-temporal
    const rsrc_t r_yp = make_rsrc(a.y_prev + tile0 * T * N, (uint32_t)(BM * N * 4));
    const rsrc_t r_yo = make_rsrc(a.y_out + tile0 * T * N, (uint32_t)(BM * N * 4));
    const uint32_t lane_off = (uint32_t)(((4 * h) * N + nw + li) * 4);
    const uint32_t row4 = (uint32_t)(N * 4);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float yp[CB][16];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t off = lane_off + (uint32_t)(32 * rb + 8 * (r >> 2) + (r & 3)) * row4 + 128 * cb;
          yp[cb][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_yp, off, 0, kNt));
        }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t off = lane_off + (uint32_t)(32 * rb + 8 * (r >> 2) + (r & 3)) * row4 + 128 * cb;
          const double d = __dmul_rn(__dmul_rn((double)acc[rb][cb][r], base), ws[cb]);
          const float y = (float)__dadd_rn((double)yp[cb][r], d);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, y), r_yo, off, 0, kNt);
        }
      // keep each row block's loads, math and stores together (bounds the
      // registers the epilogue holds at once)
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int64_t n = nw + 32 * cb + li;
      if (n >= N) continue;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int i = (32 * rb) / T;
        if (!eligible[i]) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t grow = tile0 * T + 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
          if (grow >= a.rows) continue;
          const int64_t idx = grow * N + n;
          const double d = __dmul_rn(__dmul_rn((double)acc[rb][cb][r], base), ws[cb]);
          a.y_out[idx] = (float)__dadd_rn((double)a.y_prev[idx], d);
        }
      }
    }
  }

  // ---- Ineligible tiles: exact scalar path over the FPoT groups in perm
  // order, int32 group sums shifted into int64.  Thread = one column.
  for (int i = 0; i < tiles_here; ++i) {
    if (eligible[i]) continue;
    const int64_t tau = tile0 + i;
    const int64_t n = n0 + tid;
    if (n >= N) continue;
    const int32_t* off = off_s + i * (kBins + 1);
    const uint16_t* pm = a.perm + tau * K;
    const int8_t* cd = a.codes + tau * K * T;
    const double wsn = (double)a.w_scale[n];
    for (int t0 = 0; t0 < T; t0 += 32) {
      int64_t sum[32];
#pragma unroll
      for (int t = 0; t < 32; ++t) sum[t] = 0;
      for (int g = 0; g < kTags; ++g) {
        const int lo = off[4 * g], hi = off[4 * g + 4];
        if (lo == hi) continue;
        int32_t gs[32];
#pragma unroll
        for (int t = 0; t < 32; ++t) gs[t] = 0;
        for (int j = lo; j < hi; ++j) {
          const int64_t k = pm[j];
          const int32_t wv = (int32_t)a.w[k * N + n];
          const int4* c4 = reinterpret_cast<const int4*>(cd + k * T + t0);
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            const int4 c = c4[v];
            const int words[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int b = 0; b < 16; ++b) gs[16 * v + b] += (int32_t)(int8_t)(words[b >> 2] >> (8 * (b & 3))) * wv;
          }
        }
#pragma unroll
        for (int t = 0; t < 32; ++t) sum[t] += (int64_t)gs[t] << (DSTAR_FMDQ_TAG_OFFSET - g);
      }
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        const int64_t grow = tau * T + t0 + t;
        if (grow >= a.rows) continue;
        const int64_t idx = grow * N + n;
        const double d = __dmul_rn(__dmul_rn((double)sum[t], base), wsn);
        a.y_out[idx] = (float)__dadd_rn((double)a.y_prev[idx], d);
      }
    }
  }
}

template <int T, bool VecW>
int launch_tv(const LinearArgs& a, hipStream_t s) {
  const int64_t nt = n_tiles(a.rows, T);
  const int64_t row_blocks = (nt + Cfg<T>::kTiles - 1) / Cfg<T>::kTiles;
  const int32_t col_blocks = (int32_t)((a.N + BN - 1) / BN);
  const int64_t grid = row_blocks * col_blocks;
  if (grid > 0x7FFFFFFF || row_blocks > 0x7FFFFFFF)
    return set_error(DSTAR_EUNSUPPORTED, "fmdq_linear: grid too large");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)linear_mfma_kernel<T, VecW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess)
      return set_error(DSTAR_EHIP, "fmdq_linear: hipFuncSetAttribute: %s", hipGetErrorString(e));
    attr_set = true;
  }
  hipLaunchKernelGGL((linear_mfma_kernel<T, VecW>), dim3((unsigned)grid), dim3(kThreads), kLdsBytes, s,
                     a, (int32_t)row_blocks, col_blocks);
  return check_launch("fmdq_linear (mfma)");
}

template <int T>
int launch_t(const LinearArgs& a, hipStream_t s) {
  return (a.N % 16) == 0 ? launch_tv<T, true>(a, s) : launch_tv<T, false>(a, s);
}

}  // namespace

// Handles token tiles of 32 or 64 rows, K a multiple of 64 (whole dense
// chunks) and W below 2^31 bytes (32-bit buffer offsets), given the aligned
// codes and W^T.
bool linear_mfma_supported(const LinearArgs& a) {
  return a.acodes != nullptr && a.w_t != nullptr && (a.T == 32 || a.T == 64) && (a.K % 64) == 0 &&
         (int64_t)a.K * a.N < (int64_t(1) << 31);
}

int launch_linear_mfma(const LinearArgs& a, hipStream_t s) {
  switch (a.T) {
    case 32: return launch_t<32>(a, s);
    case 64: return launch_t<64>(a, s);
    default: return set_error(DSTAR_EUNSUPPORTED, "fmdq_linear (mfma): token_tile %d", a.T);
  }
}

}  // namespace dstar
