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
// their own FPoT groups: after the dense GEMM, each 32-row block gathers its
// token tile's such channels and multiplies them group after group, in
// ascending FPoT, into a temporary int32 accumulator that is shifted left by
// the FPoT difference at every group change — the Horner form of the shift
// alignment of §3.1 step 5 and Fig. 6 — and finally added, shifted to units
// of the base, to the dense sum.
//
// Exactness.  int32 arithmetic wraps modulo 2^32 (shifts and adds included),
// so the final accumulator equals S whenever |S| < 2^31; |W| ≤ 128 (any
// int8, −128 included) gives |S| ≤ 128 · Σ_k 2^PoT_k, so a token tile is
// handled here only if 128 · Σ_k 2^PoT_k < 2^31 (computed from stage 2's bin
// counts).  Any other tile ("ineligible") is finished by an exact scalar path
// in the same workgroup: int64 sums of every channel's aligned value, rebuilt
// from the aligned codes and digit planes while walking perm bin by bin
// (aligned_tile_sums).  Neither path reads the plain codes.
//
// Stage 2 orders each FPoT group widest precision first, so the channels of a
// group with PoT ≥ 7 are a prefix of the group in perm, found from the bin
// offsets alone.
//
// Layout.  Workgroup = 256 threads = 4 waves, output block 128 rows × 256
// columns; wave w owns all 128 rows and columns 64w .. 64w+63 (4 × 2 MFMA
// 32x32x32 int8 tiles).  Grids that would give the CUs fewer workgroups than
// there are CUs use blocks of 128 × 128 instead (wave w: columns 32w ..
// 32w+31, 4 × 1 tiles; half the W bytes per stage, so the dense ring holds
// four stages instead of three).  Dense part: 64-channel chunks of stage 1's
// aligned codes ([rows][K]) and of W^T ([N][K]), both channel innermost, flow
// through a 3-stage LDS ring filled by direct global-to-LDS buffer loads; a chunk's
// stage is refilled as soon as every wave holds the fragments of its second
// k-step, so three chunks are in flight, and each k-step's six fragment reads
// are interleaved with the previous k-step's MFMAs.  The four 16-byte columns
// of every 64-byte row are XOR-swizzled by (row / 4) mod 4 so that one
// ds_read_b128 per fragment is free of bank conflicts.  The aligned-code rows
// are shared by the four waves, each wave reads only its own 64 W^T rows.
// Gathered part (digits of the channels with PoT ≥ 7): one "unit" is 64
// channels of one 32-row block's digit list; their digit codes (32 bytes per
// channel from the [tile][K][T] digit planes) and W rows (256 bytes per
// channel) are gathered by direct global-to-LDS loads into a 4-stage ring,
// three units ahead; the channel ids of up to 32 units at a time are staged
// in LDS.  Both tiles have the channel outermost, so each lane assembles its
// fragment with two ds_read_b64_tr_b8 transpose reads (W rows XOR-swizzled in
// 16-byte pieces by channel mod 8).  A workgroup whose second-digit units
// would outnumber its dense chunks (tiles where most channels have PoT ≥ 7)
// runs those digits instead as one dense pass over K, masked to its
// sub-channels with PoT ≥ 7, before the dense loop.  The bin offsets and the
// unit schedule are read while the first dense chunks are in flight.
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
constexpr int WN = 64;             // output columns per wave (the wide blocks)
constexpr int BN = kWaves * WN;    // output columns per workgroup (256; the LDS regions are sized for it)
constexpr int RB = BM / 32;        // 32-row MFMA blocks per wave (4)
constexpr int BK = 64;             // channels per dense chunk (2 MFMA k-steps)
constexpr int KS = 32;             // channels per MFMA k-step (= per gathered unit)
constexpr int kTags = DSTAR_FMDQ_NUM_TAGS;
constexpr int kBins = DSTAR_FMDQ_NUM_BINS;
constexpr int kAlignedPotMax = 6;  // q·2^e fits int8 when PoT ≤ 6
constexpr int kTwoDigitPotMax = 13;  // q·2^e needs no third digit when PoT ≤ 13
constexpr uint64_t kBoundLimit = 2147483647ull / 128ull;  // Σ 2^PoT limit (|W| ≤ 128)
constexpr int kBand = 8;           // row blocks per band of the block order

template <int T>
struct Cfg {
  static constexpr int kTiles = BM / T;   // token tiles per workgroup
};

// LDS carve-up (bytes).  The data region holds either the dense ring
// (kStages stages of (A 128 rows + B 256 rows) × 64 bytes) or, after the
// dense loop, the gathered ring (kUnits stages of A 64 channels × 32 rows +
// B 64 channels × 256 columns).  Both are 72 KiB, so two workgroups fit per CU.
constexpr int kStages = 3;
constexpr int kStageDense = (BM + BN) * BK;                // 24576
constexpr int KU = 64;                                     // channels per gathered unit
constexpr int kUnitA = KU * 32;                            // 2048
constexpr int kUnitB = KU * BN;                            // 16384
constexpr int kUnitBytes = kUnitA + kUnitB;                // 18432
constexpr int kUnits = 4;                                  // gathered ring stages
constexpr int kAhead = kUnits - 1;                         // units in flight ahead
constexpr int kBatch = 32;                                 // units whose ids are staged
constexpr int kDataBytes = kStages * kStageDense;          // 73728
static_assert(kUnits * kUnitBytes == kDataBytes, "the two rings share one region");
// Per-tile metadata is sized for the most token tiles a workgroup holds (8,
// at T = 16).  The bound parts and digit-list lengths are only used before
// the first channel ids are written, so they share the ids' region.
constexpr int kMaxTiles = BM / 16;
constexpr int kOffEnt = kDataBytes;                        // uint16 [kBatch][KU] channel ids
constexpr int kOffBp = kOffEnt;                            // uint64 [8][16] bound parts (meta only)
constexpr int kOffRc = kOffBp + kMaxTiles * kTags * 8;     // int32 [2][8][16] digit-list lengths (meta only)
static_assert(kOffRc + 2 * kMaxTiles * kTags * 4 <= kOffEnt + kBatch * KU * 2, "meta fits the ids region");
constexpr int kOffOff = kOffEnt + kBatch * KU * 2;         // int32 [8][65] bin offsets
constexpr int kOffRs = kOffOff + kMaxTiles * (kBins + 1) * 4;  // int32 [8][16] group starts in perm
constexpr int kOffPre = kOffRs + kMaxTiles * kTags * 4;    // int32 [2][8][17] list prefix sums
constexpr int kOffUs = kOffPre + 2 * kMaxTiles * 17 * 4;   // int32 [17] (+pad) unit starts
constexpr int kOffUi = kOffUs + 20 * 4;                    // uint32 [kBatch] unit tile/rows/plane
constexpr int kOffElig = kOffUi + kBatch * 4;              // int32 [8]
constexpr int kLdsBytes = kOffElig + kMaxTiles * 4;
static_assert(2 * kLdsBytes <= 160 * 1024, "two workgroups per CU");

// Operand loads go through buffer resources: a load whose offset lies outside
// the resource's byte range returns zeros, so every load is unconditional
// (an invalid piece is given the offset kOob) and the compiler can count the
// loads still in flight instead of waiting for all of them.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void* lds_ptr;
constexpr uint32_t kOob = 0x80000000u;

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; the counters not waited on at their maximum).
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }
constexpr int kWaitVm0 = wait_vm(0);
constexpr int kWaitLgkm0 = 0xC07F;         // lgkmcnt(0)

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Workgroup barrier that waits only for this wave's LDS accesses (not for
// the direct-to-LDS loads in flight, which __syncthreads would also drain).
__device__ __forceinline__ void bar_lds() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// ds_read_b64_tr_b8 issued as inline assembly: the compiler cannot tell what
// the intrinsic reads, so it would wait for every direct-to-LDS load in
// flight before it.  The caller waits (lgkm_wait) before using the result.
__device__ __forceinline__ v2i tr8(const uint8_t* p) {
  v2i r;
  const uint32_t addr = (uint32_t)(uintptr_t)(lds_ptr)p;
  __asm__ __volatile__("ds_read_b64_tr_b8 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
// Waits for this wave's LDS reads; the fragments pass through the statement
// so that no use of them can be scheduled before it.
__device__ __forceinline__ void lgkm_wait(v4i& x, v4i& y, v4i& z) {
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)" : "+v"(x), "+v"(y), "+v"(z));
}

// MFMA fragment from a [channel][row] LDS tile with row stride S: the lane
// gets row/column (lane % 32) and channels 16·(lane / 32) + 0..15.  Two
// transpose reads; in each 16-lane group, lane r addresses channel row r/2 (+8
// for the second read) at column offset 8·(r % 2) (+16 for the odd groups).
template <int S>
__device__ __forceinline__ v4i tr_frag(const uint8_t* tile, int col0, int lane) {
  const int q = lane >> 4, r = lane & 15;
  const uint8_t* p = tile + (16 * (q >> 1) + (r >> 1)) * S + col0 + 16 * (q & 1) + 8 * (r & 1);
  const v2i lo = tr8(p);
  const v2i hi = tr8(p + 8 * S);
  return v4i{lo[0], lo[1], hi[0], hi[1]};
}

// The same from a gathered W tile [32 channels][NB columns] (NB = 256 or
// 128) whose 16-byte pieces are stored XOR-swizzled: column piece P of
// channel c sits at piece P ^ (c mod 8), so the 8 channels one 16-lane group
// reads hit 8 different pieces (no bank conflicts).  Channels c and c + 8
// share the swizzle.
template <int NB>
__device__ __forceinline__ v4i tr_frag_wsw(const uint8_t* tile, int col0, int lane) {
  const int q = lane >> 4, r = lane & 15;
  const int c = 16 * (q >> 1) + (r >> 1);
  const int piece = ((col0 >> 4) + (q & 1)) ^ (c & 7);
  const uint8_t* p = tile + c * NB + 16 * piece + 8 * (r & 1);
  const v2i lo = tr8(p);
  const v2i hi = tr8(p + 8 * NB);
  return v4i{lo[0], lo[1], hi[0], hi[1]};
}

__device__ __forceinline__ void shift_acc(v16i& acc, int s) {
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = (int)((uint32_t)acc[r] << s);
}

// Gelu: the epilogue also stores GELU(Y_t) (a separate instantiation, so the
// plain kernel carries none of its code).
// WNt: output columns per wave, 64 (blocks of 128 × 256) or 32 (128 × 128,
// for grids that would leave CUs without a workgroup; 16-byte W loads only).
template <int T, bool VecW, bool Gelu, int WNt>
__global__ __launch_bounds__(kThreads, 2) void linear_mfma_kernel(LinearArgs a, int32_t row_blocks,
                                                                  int32_t col_blocks) {
  constexpr int WN = WNt;                 // output columns per wave
  constexpr int BN = kWaves * WN;         // output columns per workgroup
  constexpr int CB = WN / 32;             // 32-column MFMA blocks per wave
  static_assert(WN == 64 || (WN == 32 && VecW), "column widths");
  constexpr int kNB1 = WN / 16;           // W^T loads per wave and dense chunk (16 rows each)
  constexpr int kStageDenseT = (BM + BN) * BK;
  // Dense ring stages: the narrow blocks' stages are half the size, so their
  // ring is one stage deeper (more chunks in flight where a CU often holds a
  // single workgroup).
  constexpr int kStagesT = WN == 64 ? kStages : 4;
  constexpr int kUnitBT = KU * BN;
  constexpr int kUnitBytesT = kUnitA + kUnitBT;
  static_assert(kStagesT * kStageDenseT <= kDataBytes && kUnits * kUnitBytesT <= kDataBytes, "rings fit");
  // Waits of the dense loops, in loads per wave (L per chunk; loads complete
  // in order): chunk c + 1 has landed once at most the later kStagesT − 2
  // chunks' loads (and, in the first iterations, the eight id loads issued
  // after the first kStagesT chunks) are in flight.
  constexpr int kLChunk = 2 + kNB1;
  constexpr int kWaitVmChunkT = wait_vm((kStagesT - 2) * kLChunk);
  constexpr int kWaitVmChunkIdsT = wait_vm((kStagesT - 2) * kLChunk + 8);
  constexpr int kWaitVmFirstT = wait_vm((kStagesT - 1) * kLChunk + 8);
  static_assert((kStagesT - 1) * kLChunk + 8 <= 63, "vmcnt range");
  constexpr int kTiles = Cfg<T>::kTiles;
  // Gathered units are scheduled per (32-row block, list): per block, first
  // the third-digit lists, then the second-digit lists, of the kTPB token
  // tiles that share the block (two at T = 16, else one).
  constexpr int kTPB = T < 32 ? 32 / T : 1;
  constexpr int kSched = 2 * RB * kTPB;             // schedule entries (8 or 16)
  constexpr int kGo = (kTiles * (kBins + 1) + kThreads - 1) / kThreads;   // offset loads per thread
  // Workgroups whose second-digit lists are long (text-like tiles where most
  // channels have PoT ≥ 7) run those digits as a masked dense pass instead of
  // gathered units; written for 32-row tiles and N a multiple of 16.
  constexpr bool kDense1 = T == 32 && VecW;
  // Direct-to-LDS loads per wave per gathered unit: two dword loads of digit
  // codes, and the W rows as BN/64 16-byte or sixteen 4-byte loads.
  constexpr int kOpsUnit = VecW ? 2 + BN / 64 : 18;
  constexpr int kWaitVmUnits = wait_vm(kOpsUnit * (kAhead - 1));   // unit u landed
  static_assert(kOpsUnit * (kAhead - 1) <= 63, "vmcnt range");
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* ent = reinterpret_cast<uint16_t*>(smem + kOffEnt);         // [kBatch][KU]
  unsigned long long* bpart = reinterpret_cast<unsigned long long*>(smem + kOffBp);
  int32_t* off_s = reinterpret_cast<int32_t*>(smem + kOffOff);          // [kTiles][65]
  int32_t* rstart = reinterpret_cast<int32_t*>(smem + kOffRs);          // [kTiles][16]
  int32_t* rc = reinterpret_cast<int32_t*>(smem + kOffRc);              // [2][kTiles][16]
  int32_t* pre = reinterpret_cast<int32_t*>(smem + kOffPre);            // [2][kTiles][17]
  int32_t* ustart = reinterpret_cast<int32_t*>(smem + kOffUs);          // [kSched + 1]
  uint32_t* uinfo = reinterpret_cast<uint32_t*>(smem + kOffUi);         // [kBatch]
  int32_t* eligible = reinterpret_cast<int32_t*>(smem + kOffElig);      // [kTiles]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS bases stay scalar
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
  // This workgroup's tiles of aligned codes and perm; all of W, W^T.
  const rsrc_t r_perm = make_rsrc(a.perm + tile0 * K, (uint32_t)(tiles_here * K * 2));
  const rsrc_t r_ac = make_rsrc(a.acodes + tile0 * T * K, (uint32_t)(tiles_here * T * K));
  const rsrc_t r_w = make_rsrc(a.w, (uint32_t)(K * N));
  const rsrc_t r_wt = make_rsrc(a.w_t, (uint32_t)(N * K));

  // ---- Dense ring: every channel with PoT ≤ 6, natural order, 64 channels
  // per chunk, filled by direct global-to-LDS loads (no registers): A = the
  // 128 rows of aligned codes, shared by the four waves; B = each wave's 64
  // columns of W^T.  Both tiles are [row][64 channels] with the 16-byte
  // columns XOR-swizzled by row, (column ^ (row / 4) % 4), so the fragment
  // reads (one ds_read_b128) are free of bank conflicts.  A direct load
  // writes lane l's 16 bytes at base + 16·l: one wave instruction fills 16
  // rows.  Each wave issues 2 A and 4 B instructions per chunk.
  auto stageA = [&](int st) { return smem + st * kStageDenseT; };
  auto stageB = [&](int st, int w) { return smem + st * kStageDenseT + BM * BK + w * WN * BK; };
  const int r16 = lane >> 2;                       // row of this lane within a 16-row group
  const int c16 = (lane & 3) ^ ((r16 >> 2) & 3);   // global 16-byte column it loads
  // K a multiple of 16: the last chunk may hold fewer than 64 channels; a
  // lane whose 16-byte column starts at K loads from the out-of-range offset,
  // which writes zeros into LDS, so those columns add nothing.
  const int64_t nchunks = (K + BK - 1) / BK;
  auto issue = [&](int64_t c, int st) {
    const int64_t k0 = c * BK;
    const bool live = c < nchunks && k0 + 16 * c16 < K;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 16 * (2 * wave + j) + r16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_ac, (lds_ptr)(stageA(st) + 1024 * (2 * wave + j)), 16,
                                               live ? (uint32_t)(row * K + k0 + 16 * c16) : kOob, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kNB1; ++j) {
      const int64_t n = nw + 16 * j + r16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_wt, (lds_ptr)(stageB(st, wave) + 1024 * j), 16,
                                               live && n < N ? (uint32_t)(n * K + k0 + 16 * c16) : kOob, 0, 0, 0);
    }
  };

  // ---- Meta, overlapped with the first dense chunks: per tile and FPoT
  // group the prefixes of the group (in perm) whose channels have PoT ≥ 7
  // (second digit) and PoT ≥ 14 (third digit), the exactness bound
  // Σ_k 2^PoT_k, and the schedule of gathered units: per 32-row block the
  // third-digit list, then the second-digit list (each the concatenation of
  // the tile's group prefixes), 64 channels per unit.
  // (Unconditional loads: the compiler then waits for exactly these, not for
  // the dense loads issued after them.)
  const rsrc_t r_off = make_rsrc(a.group_off + tile0 * (kBins + 1), (uint32_t)(tiles_here * (kBins + 1) * 4));
  uint32_t go[kGo];
#pragma unroll
  for (int m = 0; m < kGo; ++m) {
    const int idx = tid + kThreads * m;
    go[m] = __builtin_amdgcn_raw_buffer_load_b32(r_off, idx < kTiles * (kBins + 1) ? (uint32_t)(4 * idx) : kOob, 0, 0);
  }
  __asm__ __volatile__("" ::: "memory");   // keep these loads ahead of the dense ones
#pragma unroll
  for (int c = 0; c < kStagesT; ++c) issue(c, c);   // a chunk past K loads zeros
#pragma unroll
  for (int m = 0; m < kGo; ++m) {
    const int idx = tid + kThreads * m;
    if (idx < kTiles * (kBins + 1)) off_s[idx] = (int32_t)go[m];
  }
  bar_lds();
  if (tid < kTiles * kTags) {
    const int i = tid / kTags, g = tid % kTags;
    const int e = DSTAR_FMDQ_TAG_OFFSET - g;
    const int32_t* o = off_s + i * (kBins + 1);
    // PoT = e + 2·pc.  Bins of group g run from precision code 3 (bin 4g)
    // down to 0 (bin 4g + 3), so the channels with pc ≥ pcmin are the first
    // o[4g + 4 − pcmin] − o[4g] of the group.
    const int pc7 = max(0, (kAlignedPotMax + 2 - e) / 2);     // PoT ≥ 7
    const int pc14 = max(0, (kTwoDigitPotMax + 2 - e) / 2);   // PoT ≥ 14
    rstart[tid] = o[4 * g];
    rc[tid] = pc7 <= 3 ? o[4 * g + 4 - pc7] - o[4 * g] : 0;
    rc[kTiles * kTags + tid] = pc14 <= 3 ? o[4 * g + 4 - pc14] - o[4 * g] : 0;
    unsigned long long b = 0;
#pragma unroll
    for (int pc = 0; pc < 4; ++pc)
      b += (unsigned long long)(o[4 * g + 4 - pc] - o[4 * g + 3 - pc]) << (e + 2 * pc);
    bpart[tid] = b;
  }
  bar_lds();
  if (tid < kTiles * 16) {
    // thread = 16 · tile + group (up to two waves; a tile's 16 threads sit in
    // one wave)
    const int i = tid >> 4, g = tid & 15;
    unsigned long long b = 0;
    for (int g2 = 0; g2 < kTags; ++g2) b += bpart[i * kTags + g2];
    const bool el = i < tiles_here && b <= kBoundLimit;
    if (g == 0) eligible[i] = el ? 1 : 0;
    // Inclusive prefix sums of both list lengths over the tile's groups.
    int s0 = rc[tid], s1 = rc[kTiles * kTags + tid];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int n0 = __shfl_up(s0, o, 16), n1 = __shfl_up(s1, o, 16);
      if (g >= o) {
        s0 += n0;
        s1 += n1;
      }
    }
    pre[i * 17 + g + 1] = s0;
    pre[kTiles * 17 + i * 17 + g + 1] = s1;
    if (g == 0) {
      pre[i * 17] = 0;
      pre[kTiles * 17 + i * 17] = 0;
    }
  }
  bar_lds();
  if (wave == 0) {
    // Unit starts: an exclusive scan over the schedule entries x: block
    // rb = x / (2·kTPB), entry e = x % (2·kTPB); e < kTPB is the third-digit
    // list (plane 1) of the block's tile e, the rest the second-digit lists
    // (plane 0).
    const int x = lane;
    const int rb = x / (2 * kTPB), e = x % (2 * kTPB);
    const int lvl = e < kTPB ? 1 : 0;
    const int ti = T < 32 ? rb * kTPB + e % kTPB : (32 * rb) / T;
    int v = 0;
    if (x < kSched && eligible[ti]) v = (pre[lvl * kTiles * 17 + ti * 17 + 16] + KU - 1) / KU;
    if constexpr (kDense1) {
      // More second-digit units than dense chunks: a dense pass over all K
      // channels (masked to the sub-channels with PoT ≥ 7) does less work, so
      // the second-digit lists leave the schedule (K ≤ 8192: the mask's
      // bitmap fits the id region).
      int u1 = lvl == 0 ? v : 0;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) u1 += __shfl_xor(u1, o, 64);
      const bool d1 = u1 > nchunks && K <= 8192;
      if (d1 && lvl == 0) v = 0;
      if (lane == 0) ustart[19] = d1 ? 1 : 0;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int n = __shfl_up(v, o, 64);
      if (lane >= o) v += n;
    }
    if (lane < kSched) ustart[lane + 1] = v;
    if (lane == 0) ustart[0] = 0;
  }
  bar_lds();
  const int U = ustart[kSched];   // gathered units of this workgroup

  // Channel ids of units [ubase, ubase + kBatch): thread → (unit, 8 ids).
  // fetch() issues the loads into registers, commit() writes them to LDS.
  uint32_t fid[8], fok, finfo;
  auto fetch = [&](int ubase) __attribute__((always_inline)) {
    const int uu = ubase + (tid >> 3), q8 = tid & 7;
    int x = 0;
#pragma unroll
    for (int st = 8; st >= 1; st >>= 1)   // largest x with ustart[x] <= uu
      if (x + st < kSched && ustart[x + st] <= uu) x += st;
    const bool valid = uu < U;
    const int rb = x / (2 * kTPB), e = x % (2 * kTPB);
    const int lvl = e < kTPB ? 1 : 0;
    const int i = T < 32 ? rb * kTPB + e % kTPB : (32 * rb) / T;
    // which part of the unit's 32 rows the tile fills (T = 16: its half), or
    // which 32 rows of the tile the unit covers (T = 64)
    const int sub = T < 32 ? e % kTPB : rb % (T / 32 > 0 ? T / 32 : 1);
    const int32_t* pr = pre + lvl * kTiles * 17 + i * 17;
    const int total = valid ? pr[16] : 0;
    int pos = KU * (uu - ustart[x]) + 8 * q8;
    int g = 0;
#pragma unroll
    for (int st = 8; st >= 1; st >>= 1)   // group of pos: largest g with pr[g] <= pos
      if (g + st < kTags && pr[g + st] <= pos) g += st;
    // (The loaded ids are only touched in commit(), so the loads stay in
    // flight until then.)
    fok = 0;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj, ++pos) {
      while (g + 1 < kTags && pr[g + 1] <= pos) ++g;
      const bool ok = pos < total;
      const uint32_t off = ok ? (uint32_t)(((int64_t)i * K + rstart[i * kTags + g] + (pos - pr[g])) * 2) : kOob;
      fid[jj] = __builtin_amdgcn_raw_buffer_load_b16(r_perm, off, 0, 0);
      fok |= (ok ? 1u : 0u) << jj;
    }
    finfo = (uint32_t)i | ((uint32_t)sub << 3) | ((uint32_t)lvl << 4);
  };
  auto commit = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) fid[jj] = ((fok >> jj) & 1u) ? (fid[jj] & 0xFFFFu) : 0xFFFFu;
    uint4 p;
    p.x = fid[0] | (fid[1] << 16);
    p.y = fid[2] | (fid[3] << 16);
    p.z = fid[4] | (fid[5] << 16);
    p.w = fid[6] | (fid[7] << 16);
    *reinterpret_cast<uint4*>(ent + (tid >> 3) * KU + 8 * (tid & 7)) = p;
    if ((tid & 7) == 0) uinfo[tid >> 3] = finfo;
  };

  v16i acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0;

  // The ids of the first gathered units are loaded now and held in registers
  // through the dense loop (eight loads, issued even when there is no unit,
  // so that the loop's first two waits can count them).
  fetch(0);
  __asm__ __volatile__("" ::: "memory");

  // ---- Masked dense pass over the second digits (workgroups chosen above).
  // Horner order of the shift alignment: acc = Σ_k d1·W over the sub-channels
  // with PoT ≥ 7, then acc ·= 2^7, the dense loop below adds Σ_k d0·W, and
  // the gathered third digits are added ·2^15.  First a bitmap of those
  // sub-channels is built in the id region (one bit per (tile, channel),
  // K ≤ 8192; the region is free until the ids are committed) from the
  // second-digit prefixes of the FPoT groups, read from the tiles' perm rows
  // staged in the ring.  Then chunks of 64 channels flow through the ring as
  // in the dense loop: A = each tile's [64 channels][32 rows] block of digit
  // plane 0 (wave w loads tile w's), a sub-channel's 32 bytes loaded only if
  // its bit is set (that plane is unwritten elsewhere); B = the chunk of W^T.
  const bool dense1 = kDense1 && ustart[19] != 0;
  if constexpr (kDense1) {
    if (dense1) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the first dense chunks and the ids
      bar_lds();                              // every wave past the meta phase
      const int kw = (int)((K + 31) / 32);    // bitmap words per tile
      uint32_t* bm = reinterpret_cast<uint32_t*>(smem + kOffEnt);   // [kTiles][kw]
      const uint16_t* pst = reinterpret_cast<const uint16_t*>(smem);   // [tiles][K] staged perm
      for (int q = tid; q < kTiles * kw; q += kThreads) bm[q] = 0u;
      const int pbytes = (int)(kTiles * K * 2);
      for (int b0 = 0; b0 < pbytes; b0 += kThreads * 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r_perm, (lds_ptr)(smem + b0 + 1024 * wave), 16,
                                                 (uint32_t)(b0 + 16 * tid), 0, 0, 0);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      bar_lds();
      for (int i = 0; i < tiles_here; ++i) {
        if (!eligible[i]) continue;
        for (int g = 0; g < kTags; ++g) {
          const int lo = rstart[i * kTags + g];
          const int n = pre[i * 17 + g + 1] - pre[i * 17 + g];   // the group's PoT ≥ 7 prefix
          for (int q = tid; q < n; q += kThreads) {
            const uint32_t k = pst[i * K + lo + q];
            atomicOr(&bm[i * kw + (int)(k >> 5)], 1u << (k & 31u));
          }
        }
      }
      bar_lds();
      const rsrc_t r_d1 = make_rsrc(a.hcodes + tile0 * K * T, (uint32_t)(tiles_here * K * T));
      const uint32_t* bmw = bm + wave * kw;
      auto issue1 = [&](int64_t c, int st) __attribute__((always_inline)) {
        const int64_t k0 = c * BK;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t k = k0 + 32 * j + (lane >> 1);   // lane pair → one sub-channel's 32 bytes
          const bool in = c < nchunks && k < K;
          const bool ok = in && ((bmw[in ? (int)(k >> 5) : 0] >> (k & 31)) & 1u);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              r_d1, (lds_ptr)(stageA(st) + 2048 * wave + 1024 * j), 16,
              ok ? (uint32_t)((wave * K + k) * T + 16 * (lane & 1)) : kOob, 0, 0, 0);
        }
        const bool live = c < nchunks && k0 + 16 * c16 < K;
#pragma unroll
        for (int j = 0; j < kNB1; ++j) {
          const int64_t n = nw + 16 * j + r16;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r_wt, (lds_ptr)(stageB(st, wave) + 1024 * j), 16,
                                                   live && n < N ? (uint32_t)(n * K + k0 + 16 * c16) : kOob, 0, 0,
                                                   0);
        }
      };
      struct Frags1 { v4i a[RB], b[CB]; };
      auto read1 = [&](Frags1& f, int st, int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int row = 32 * cb + li, cc = 2 * ks + h;
          f.b[cb] = *reinterpret_cast<const v4i*>(stageB(st, wave) + row * BK + 16 * (cc ^ ((row >> 2) & 3)));
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) f.a[rb] = tr_frag<32>(stageA(st) + 2048 * rb + KS * 32 * ks, 0, lane);
      };
      // the transpose reads are inline assembly: wait for them by hand
      auto wait1 = [&](Frags1& f) __attribute__((always_inline)) {
        __asm__ __volatile__("s_waitcnt lgkmcnt(0)" : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]));
      };
      auto mma1 = [&](const Frags1& f) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.a[rb], f.b[cb], acc[rb][cb], 0, 0, 0);
      };
#pragma unroll
      for (int c = 0; c < kStagesT; ++c) issue1(c, c);
      __builtin_amdgcn_s_waitcnt(wait_vm((kStagesT - 1) * kLChunk));  // chunk 0
      __asm__ __volatile__("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ __volatile__("" ::: "memory");
      Frags1 g0, g1;
      read1(g0, 0, 0);
      for (int64_t c = 0; c < nchunks; ++c) {
        const int st = (int)(c % kStagesT);
        const int st1 = (int)((c + 1) % kStagesT);
        wait1(g0);
        mma1(g0);
        read1(g1, st, 1);
        __builtin_amdgcn_s_waitcnt(kWaitVmChunkT);   // chunk c + 1 (chunk c + 2 after it)
        bar_lds();                                   // also completes g1's reads
        issue1(c + kStagesT, st);
        wait1(g1);
        mma1(g1);
        read1(g0, st1, 0);
      }
      wait1(g0);                                // the last (unused) reads
      __builtin_amdgcn_s_waitcnt(kWaitVm0);     // the chunks issued past K
      bar_lds();                                // every wave done with the ring and the bitmap
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) shift_acc(acc[rb][cb], 7);
      // The dense loop's first chunks again, then the ids again: the same
      // loads in flight, in the same order, as its waits count.
#pragma unroll
      for (int c = 0; c < kStagesT; ++c) issue(c, c);
      fetch(0);
      __asm__ __volatile__("" ::: "memory");
    }
  }

  // ---- Dense loop.
  {
    auto frag = [&](const uint8_t* tile, int row, int c) {
      return *reinterpret_cast<const v4i*>(tile + row * BK + 16 * (c ^ ((row >> 2) & 3)));
    };
    // One k-step's fragments: 4 row blocks of codes, 2 column blocks of W^T.
    struct Frags { v4i a[RB], b[CB]; };
    auto read = [&](Frags& f, int st, int ks) __attribute__((always_inline)) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) f.b[cb] = frag(stageB(st, wave), 32 * cb + li, 2 * ks + h);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) f.a[rb] = frag(stageA(st), 32 * rb + li, 2 * ks + h);
    };
    // The MFMAs of one k-step with the six fragment reads of the next one
    // interleaved (one read after each of the first six MFMAs), so the reads
    // are in flight while the matrix core works.
    auto mma = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.a[rb], f.b[cb], acc[rb][cb], 0, 0, 0);
      constexpr int kPairs = RB * CB < RB + CB ? RB * CB : RB + CB;
#pragma unroll
      for (int i = 0; i < kPairs; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      }
      if constexpr (RB * CB > kPairs) __builtin_amdgcn_sched_group_barrier(0x008, RB * CB - kPairs, 0);
      if constexpr (RB + CB > kPairs) __builtin_amdgcn_sched_group_barrier(0x100, RB + CB - kPairs, 0);
    };
    // Chunk c's stage is free once every wave holds its second k-step's
    // fragments, so the wait for chunk c + 1 and the barrier sit between the
    // two k-steps of chunk c, and chunk c + kStagesT is issued into that stage
    // right after: kStagesT chunks are in flight.  Chunks past K load zeros
    // (their fragments are read but never used), so every wait has the same
    // count; in the first kStagesT − 1 waits the eight id loads (issued after
    // the first kStagesT chunks) may also be in flight.
    Frags f0, f1;
    __builtin_amdgcn_s_waitcnt(kWaitVmFirstT);
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
    read(f0, 0, 0);
    for (int64_t c = 0; c < nchunks; ++c) {
      const int st = (int)(c % kStagesT);
      const int st1 = (int)((c + 1) % kStagesT);
      read(f1, st, 1);
      mma(f0);
      if (c < kStagesT - 1) {
        __builtin_amdgcn_s_waitcnt(kWaitVmChunkIdsT);
      } else {
        __builtin_amdgcn_s_waitcnt(kWaitVmChunkT);
      }
      bar_lds();
      issue(c + kStagesT, st);
      read(f0, st1, 0);
      mma(f1);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the chunks issued past K
  }

  // ---- Epilogue set-up.  Y is streamed once: its loads and stores are
  // non-temporal so they do not evict W and the codes from the caches.  In
  // interior blocks the epilogue runs over (32-row block, 32-column block)
  // units, loading the Y_{t−1} of the two next units before storing the
  // current one.
  // Offsets are 32-bit, relative to this workgroup's first row.
  const double base = a.base_dev != nullptr ? (double)*a.base_dev : a.base;
  bool all_eligible = true;
#pragma unroll
  for (int i = 0; i < kTiles; ++i) all_eligible = all_eligible && eligible[i];
  const bool interior = all_eligible && (tile0 * T + BM <= a.rows) && (nw + WN <= N);
  constexpr int kNt = 2;   // aux bit: non-temporal
  const rsrc_t r_yp = make_rsrc(a.y_prev + tile0 * T * N, (uint32_t)(BM * N * 4));
  const rsrc_t r_yo = make_rsrc(a.y_out + tile0 * T * N, (uint32_t)(BM * N * 4));
  constexpr bool has_gelu = Gelu;
  const rsrc_t r_go = make_rsrc(Gelu ? a.gelu_out + tile0 * T * N : a.y_out, (uint32_t)(BM * N * 4));
  const uint32_t lane_off = (uint32_t)(((4 * h) * N + nw + li) * 4);
  const uint32_t row4 = (uint32_t)(N * 4);
  auto y_off = [&](int rb, int cb, int r) {
    return lane_off + (uint32_t)(32 * rb + 8 * (r >> 2) + (r & 3)) * row4 + 128 * cb;
  };
  float ypa[16], ypb[16], ypc[16];
  auto load_y = [&](float (&dst)[16], int rb, int cb) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      dst[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_yp, y_off(rb, cb, r), 0, kNt));
  };

  // ---- Channels with PoT ≥ 7, per 32-row block: their second digits
  // (and, for PoT ≥ 14, third digits) times W, added to the dense sum at
  // shifts 7 and 15.  Unit v (64 channels of one list) occupies ring stage
  // v % kUnits: A = [64 channels][32 rows] digit codes, B = [64 channels][256
  // columns] of W, swizzled.  Each wave loads 512 bytes of A (dword loads:
  // channel 8·m + lane/8, dword lane % 8, for its two m) and a quarter of B.
  // Every step issues exactly one unit (past the end of the list its loads
  // read nothing and write zeros into a free stage), so every wait is the
  // same count.  Columns past N only feed outputs that are never stored.
  if (U > 0) {
    commit();
    bar_lds();   // ids visible; every wave is done with the dense ring
    int ubase = 0, u = 0;
    // Unit starts: lane x holds ustart[x] (x ≤ kSched), read with readlane.
    const int us_lane = ustart[min(lane, kSched)];
    auto us_at = [&](int x) -> int { return __builtin_amdgcn_readlane(us_lane, x); };
    // Both digit planes of this workgroup's tiles through one resource: the
    // second plane starts plane_off bytes after the first (n_t·K·T < 2^31).
    const uint32_t plane_off = (uint32_t)(nt * K * T);
    const rsrc_t r_h = make_rsrc(a.hcodes + tile0 * K * T, plane_off + (uint32_t)(tiles_here * K * T));
    // The ids one wave needs for one unit's loads (all LDS reads first, so
    // they share one wait).
    // W rows: with 16-byte loads one 1 KB load holds kCh channels' row
    // segments (BN bytes each), kLpc lanes per channel.
    constexpr int kNB = VecW ? BN / 64 : 16;
    constexpr int kCh = 1024 / BN, kLpc = BN / 16;
    struct UnitIds {
      uint32_t inf, chA[2], chB[kNB];
    };
    auto load_ids = [&](int v, UnitIds& d) __attribute__((always_inline)) {
      const int vb = min(v - ubase, kBatch - 1);
      const uint16_t* en = ent + vb * KU;
      d.inf = uinfo[vb];
#pragma unroll
      for (int m = 0; m < 2; ++m) d.chA[m] = en[8 * (2 * wave + m) + (lane >> 3)];
#pragma unroll
      for (int m = 0; m < kNB; ++m)
        d.chB[m] = VecW ? en[kCh * (kNB * wave + m) + lane / kLpc] : en[16 * wave + m];
    };
    // The lane's fixed part of each W-row load: the 16-byte piece (VecW: of
    // 16 bytes, else a dword of it) of its channel's 256-byte row segment.
    uint32_t colB[kNB];
#pragma unroll
    for (int m = 0; m < kNB; ++m) {
      if constexpr (VecW) {
        const int c = kCh * (kNB * wave + m) + lane / kLpc;
        colB[m] = (uint32_t)(n0 + 16 * ((lane % kLpc) ^ (c & 7)));
      } else {
        const int c = 16 * wave + m;
        colB[m] = (uint32_t)(n0 + 16 * ((lane >> 2) ^ (c & 7)) + 4 * (lane & 3));
      }
    }
    const uint32_t tileKT = (uint32_t)(K * T);   // bytes of one tile's digit plane
    auto issue_ids = [&](int v, const UnitIds& d, bool live) __attribute__((always_inline)) {
      const uint32_t inf = __builtin_amdgcn_readfirstlane(d.inf);   // the same in every lane
      const int i = (int)(inf & 7u);
      const int sub = (int)((inf >> 3) & 1u);
      const uint32_t abase = ((inf & 16u) ? plane_off : 0u) + (uint32_t)i * tileKT;
      // dword of the tile's T-byte code run this lane loads (rows 4·dw ..
      // 4·dw + 3 of the run), and whether it lies in the run: at T = 16 the
      // tile fills rows 16·sub .. 16·sub + 15 of the unit and the other half
      // reads zeros; at T = 64 the unit is rows 32·sub .. 32·sub + 31 of it
      const int dw = T < 32 ? (lane & 7) - 4 * sub : (T == 64 ? 8 * sub : 0) + (lane & 7);
      const bool in_run = T < 32 ? (dw >= 0 && dw < T / 4) : true;
      uint8_t* sA = smem + (v % kUnits) * kUnitBytesT;
      uint8_t* sB = sA + kUnitA;
      // Offsets in 32 bits: ch·T + the tile's plane part < 2^31 and, with
      // ch < 2^16 and N < 2^23, ch·N is a 24-bit product below K·N < 2^31.
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int mm = 2 * wave + m;              // channels 8·mm .. 8·mm + 7
        const uint32_t ch = d.chA[m];
        const uint32_t off = abase + ch * (uint32_t)T + (uint32_t)(4 * dw);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r_h, (lds_ptr)(sA + 256 * mm), 4,
                                                 live && in_run && ch != 0xFFFFu ? off : kOob, 0, 0, 0);
      }
#pragma unroll
      for (int m = 0; m < kNB; ++m) {
        const uint32_t ch = d.chB[m];
        const uint32_t off = __umul24(ch, (uint32_t)N) + colB[m];
        const uint32_t o = live && ch != 0xFFFFu ? off : kOob;
        if constexpr (VecW) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r_w, (lds_ptr)(sB + 1024 * (kNB * wave + m)), 16, o, 0, 0, 0);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r_w, (lds_ptr)(sB + BN * (16 * wave + m)), 4, o, 0, 0, 0);
        }
      }
    };
    auto issue_unit = [&](int v) __attribute__((always_inline)) {
      UnitIds d;
      load_ids(v, d);
      issue_ids(v, d, v < min(U, ubase + kBatch));
    };
#pragma unroll
    for (int j = 0; j < kAhead; ++j) issue_unit(j);
    // One unit: wait for its loads, barrier, refill the ring, MFMA.
    auto step = [&](v16i (&tmp)[CB]) __attribute__((always_inline)) {
      if (u == ubase + kBatch) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        bar_lds();   // every wave is done with the previous ids
        ubase = u;
        fetch(ubase);
        commit();
        bar_lds();
#pragma unroll
        for (int j = 0; j < kAhead; ++j) issue_unit(u + j);
      }
      // The ids of unit u + kAhead are read before the wait (its stage is only
      // written after the barrier).
      UnitIds nx;
      load_ids(u + kAhead, nx);
      const bool live = u + kAhead < min(U, ubase + kBatch);
      __builtin_amdgcn_s_waitcnt(kWaitVmUnits);
      __asm__ __volatile__("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ __volatile__("" ::: "memory");
      issue_ids(u + kAhead, nx, live);
      const uint8_t* sA = smem + (u % kUnits) * kUnitBytesT;
      const uint8_t* sB = sA + kUnitA;
#pragma unroll
      for (int ks = 0; ks < KU / KS; ++ks) {
        v4i af = tr_frag<32>(sA + ks * KS * 32, 0, lane);
        v4i b0 = tr_frag_wsw<BN>(sB + ks * KS * BN, WN * wave, lane);
        v4i b1 = CB > 1 ? tr_frag_wsw<BN>(sB + ks * KS * BN, WN * wave + 32, lane) : b0;
        lgkm_wait(af, b0, b1);
        tmp[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, b0, tmp[0], 0, 0, 0);
        if constexpr (CB > 1) tmp[CB - 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, b1, tmp[CB - 1], 0, 0, 0);
      }
      ++u;
    };
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int x0 = 2 * kTPB * rb;
      const int n2 = us_at(x0 + kTPB) - us_at(x0);              // third-digit units
      const int n1 = us_at(x0 + 2 * kTPB) - us_at(x0 + kTPB);   // second-digit units
      if (n1 + n2 == 0) continue;
      v16i tmp[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmp[cb][r] = 0;
      for (int s = 0; s < n2 + n1; ++s) {
        if (s == n2 && n2 > 0) {   // third digits done: tmp = Σ d2·W · 2^8
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) shift_acc(tmp[cb], 8);
        }
        step(tmp);
      }
      // acc += (Σ d1·W + 2^8 Σ d2·W) · 2^7, or after the second-digit pass
      // (tmp = Σ d2·W alone) acc += tmp · 2^15
      const int sh = dense1 ? 15 : 7;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[rb][cb][r] = (int)((uint32_t)acc[rb][cb][r] + ((uint32_t)tmp[cb][r] << sh));
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the loads issued past the last unit
  }

  // ---- Optional dump of the exact integer S of the eligible tiles in
  // [dbg_lo, dbg_hi) (for checking; the ineligible ones are dumped by the
  // scalar path below).  Lane layout of a 32x32 MFMA result: row
  // 8·(r / 4) + 4·h + r % 4, column li.
  if (a.s_dbg != nullptr) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int64_t n = nw + 32 * cb + li;
        if (n >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);   // of the workgroup's rows
          const int i = row / T;
          const int64_t tau = tile0 + i;
          if (i >= tiles_here || !eligible[i] || tau < a.dbg_lo || tau >= a.dbg_hi) continue;
          a.s_dbg[((tau - a.dbg_lo) * T + row % T) * N + n] = (int64_t)acc[rb][cb][r];
        }
      }
    }
  }

  // ---- Epilogue: dequantize, add the cached output, store (float64 combine).
  double ws[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int64_t n = nw + 32 * cb + li;
    ws[cb] = n < N ? (double)a.w_scale[n] : 0.0;
  }
  if (interior) {
    // three buffers: the loads of the two next units are in flight while
    // one unit is combined and stored
    load_y(ypa, 0, 0);
    load_y(ypb, 1 / CB, 1 % CB);
#pragma unroll
    for (int v = 0; v < RB * CB; ++v) {
      const int rb = v / CB, cb = v % CB;
      float (&cur)[16] = v % 3 == 0 ? ypa : v % 3 == 1 ? ypb : ypc;
      float (&nxt)[16] = v % 3 == 0 ? ypc : v % 3 == 1 ? ypa : ypb;
      if (v + 2 < RB * CB) load_y(nxt, (v + 2) / CB, (v + 2) % CB);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const double d = __dmul_rn(__dmul_rn((double)acc[rb][cb][r], base), ws[cb]);
        const float y = (float)__dadd_rn((double)cur[r], d);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, y), r_yo, y_off(rb, cb, r), 0, kNt);
        if constexpr (has_gelu)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, gelu_of(y)), r_go, y_off(rb, cb, r), 0, kNt);
      }
      // keep each unit's loads, math and stores in this order (bounds the
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
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
          if (!eligible[row / T]) continue;
          const int64_t grow = tile0 * T + row;
          if (grow >= a.rows) continue;
          const int64_t idx = grow * N + n;
          const double d = __dmul_rn(__dmul_rn((double)acc[rb][cb][r], base), ws[cb]);
          const float y = (float)__dadd_rn((double)a.y_prev[idx], d);
          a.y_out[idx] = y;
          if constexpr (has_gelu) a.gelu_out[idx] = gelu_of(y);
        }
      }
    }
  }

  // ---- Ineligible tiles: exact int64 path over the channels in perm order,
  // from the aligned codes and digit planes.  Thread = one column.
  for (int i = 0; i < tiles_here; ++i) {
    if (eligible[i]) continue;
    const int64_t tau = tile0 + i;
    const int64_t n = n0 + tid;
    if (tid >= BN || n >= N) continue;
    const int32_t* off = off_s + i * (kBins + 1);
    const double wsn = (double)a.w_scale[n];
    constexpr int TR = T < 32 ? T : 32;   // rows per pass
    for (int t0 = 0; t0 < T; t0 += TR) {
      int64_t sum[TR];
      aligned_tile_sums<T, TR>(a, off, tau, t0, n, sum);
      if (a.s_dbg != nullptr && tau >= a.dbg_lo && tau < a.dbg_hi) {
#pragma unroll
        for (int t = 0; t < TR; ++t) a.s_dbg[((tau - a.dbg_lo) * T + t0 + t) * N + n] = sum[t];
      }
#pragma unroll
      for (int t = 0; t < TR; ++t) {
        const int64_t grow = tau * T + t0 + t;
        if (grow >= a.rows) continue;
        const int64_t idx = grow * N + n;
        const double d = __dmul_rn(__dmul_rn((double)sum[t], base), wsn);
        const float y = (float)__dadd_rn((double)a.y_prev[idx], d);
        a.y_out[idx] = y;
        if constexpr (has_gelu) a.gelu_out[idx] = gelu_of(y);
      }
    }
  }
}

template <int T, bool VecW, bool Gelu, int WNt>
int launch_tvw(const LinearArgs& a, hipStream_t s) {
  constexpr int kBN = kWaves * WNt;
  const int64_t nt = n_tiles(a.rows, T);
  const int64_t row_blocks = (nt + Cfg<T>::kTiles - 1) / Cfg<T>::kTiles;
  const int32_t col_blocks = (int32_t)((a.N + kBN - 1) / kBN);
  const int64_t grid = row_blocks * col_blocks;
  if (grid > 0x7FFFFFFF || row_blocks > 0x7FFFFFFF)
    return set_error(DSTAR_EUNSUPPORTED, "fmdq_linear: grid too large");
  // The LDS limit is a per-device property of the kernel: set it on every
  // launch (a host-side call; cheap, thread-safe, right on any device).
  hipError_t e = hipFuncSetAttribute((const void*)linear_mfma_kernel<T, VecW, Gelu, WNt>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess)
    return set_error(DSTAR_EHIP, "fmdq_linear: hipFuncSetAttribute: %s", hipGetErrorString(e));
  hipLaunchKernelGGL((linear_mfma_kernel<T, VecW, Gelu, WNt>), dim3((unsigned)grid), dim3(kThreads), kLdsBytes,
                     s, a, (int32_t)row_blocks, col_blocks);
  return check_launch("fmdq_linear (mfma)");
}

// Blocks of 128 × 256, or of 128 × 128 when the wider blocks would number
// fewer than the CUs (each workgroup then has half the work, and the slowest
// one, often a block of text tiles that runs two dense passes, finishes
// sooner).  The narrow blocks need 16-byte W loads.
template <int T, bool VecW, bool Gelu>
int launch_tv(const LinearArgs& a, hipStream_t s) {
  if constexpr (VecW) {
    const int64_t row_blocks = (n_tiles(a.rows, T) + Cfg<T>::kTiles - 1) / Cfg<T>::kTiles;
    const int64_t wide = row_blocks * ((a.N + BN - 1) / BN);
    if (wide < cu_count()) return launch_tvw<T, VecW, Gelu, 32>(a, s);
  }
  return launch_tvw<T, VecW, Gelu, 64>(a, s);
}

template <int T>
int launch_t(const LinearArgs& a, hipStream_t s) {
  if (a.gelu_out != nullptr)
    return (a.N % 16) == 0 ? launch_tv<T, true, true>(a, s) : launch_tv<T, false, true>(a, s);
  return (a.N % 16) == 0 ? launch_tv<T, true, false>(a, s) : launch_tv<T, false, false>(a, s);
}

}  // namespace

// Handles token tiles of 16, 32 or 64 rows, K a multiple of 16 (whole
// 16-byte columns of a dense chunk), W below 2^31 bytes and each digit
// plane at most 2^30 bytes (32-bit buffer offsets, with the out-of-range
// offset 2^31 past every resource), given the aligned codes and W^T.
bool linear_mfma_supported(const LinearArgs& a) {
  return a.acodes != nullptr && a.hcodes != nullptr && a.w_t != nullptr &&
         (a.T == 16 || a.T == 32 || a.T == 64) &&
         (a.K % 16) == 0 && 2 * n_tiles(a.rows, a.T) * a.K * a.T <= (int64_t(1) << 31) &&
         (int64_t)a.K * a.N < (int64_t(1) << 31) && (int64_t)a.N * 4 * BM < (int64_t(1) << 32);
}

int launch_linear_mfma(const LinearArgs& a, hipStream_t s) {
  switch (a.T) {
    case 16: return launch_t<16>(a, s);
    case 32: return launch_t<32>(a, s);
    case 64: return launch_t<64>(a, s);
    default: return set_error(DSTAR_EUNSUPPORTED, "fmdq_linear (mfma): token_tile %d", a.T);
  }
}

}  // namespace dstar
