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
// so the final accumulator equals S whenever |S| < 2^31; |S| ≤ 127 · Σ_k
// 2^PoT_k, so a token tile is handled here only if 127 · Σ_k 2^PoT_k < 2^31
// (computed from stage 2's bin counts).  Any other tile ("ineligible") is
// finished by an exact scalar path in the same workgroup that walks the
// tile's FPoT groups in perm order with int32 group sums shifted into an int64
// sum.
//
// Stage 2 orders each FPoT group widest precision first, so the channels of a
// group with PoT ≥ 7 are a prefix of the group in perm, found from the bin
// offsets alone.
//
// Layout.  Workgroup = 256 threads = 4 waves, output block 128 rows × 256
// columns; wave w owns all 128 rows and columns 64w .. 64w+63 (4 × 2 MFMA
// 32x32x32 int8 tiles).  Dense part: 64-channel chunks of stage 1's aligned
// codes ([rows][K]) and of W^T ([N][K]), both channel innermost, flow through
// a 3-stage LDS ring filled by direct global-to-LDS buffer loads, two chunks
// ahead of the MFMAs; the four 16-byte columns of every 64-byte row are
// XOR-swizzled by (row / 4) mod 4 so that one ds_read_b128 per fragment is
// free of bank conflicts.  The aligned-code rows are shared by the four waves,
// each wave reads only its own 64 W^T rows.  Gathered part: one "unit" is 32
// channels of one FPoT group for one 32-row block: their codes (32 bytes per
// channel from the [tile][K][T] layout) and their W rows (256 bytes per
// channel) are gathered by direct global-to-LDS loads into an 8-stage ring,
// seven units ahead; the channel ids of up to 64 units at a time are staged in
// LDS.  Both tiles have the channel outermost, so each lane assembles its
// fragment with two ds_read_b64_tr_b8 transpose reads (W rows XOR-swizzled in
// 16-byte pieces by channel mod 8).  The bin offsets and the unit schedule
// are read while the first dense chunks are in flight.
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
static_assert(CB == 2, "the gathered step is written for two column blocks");
constexpr int BK = 64;             // channels per dense chunk (2 MFMA k-steps)
constexpr int KS = 32;             // channels per MFMA k-step (= per gathered unit)
constexpr int kTags = DSTAR_FMDQ_NUM_TAGS;
constexpr int kBins = DSTAR_FMDQ_NUM_BINS;
constexpr int kAlignedPotMax = 6;  // q·2^e fits int8 when PoT ≤ 6
constexpr uint64_t kBoundLimit = 2147483647ull / 127ull;  // Σ 2^PoT limit
constexpr int kBand = 8;           // row blocks per band of the block order

template <int T>
struct Cfg {
  static constexpr int kTiles = BM / T;   // token tiles per workgroup
};

// LDS carve-up (bytes).  The data region holds either the dense ring
// (kStages stages of (A 128 rows + B 256 rows) × 64 bytes) or, after the
// dense loop, the gathered ring (kUnits stages of A 32 channels × 32 rows +
// B 32 channels × 256 columns).  Both are 72 KiB, so two workgroups fit per CU.
constexpr int kStages = 3;
constexpr int kStageDense = (BM + BN) * BK;                // 24576
constexpr int kUnitA = KS * 32;                            // 1024
constexpr int kUnitB = KS * BN;                            // 8192
constexpr int kUnitBytes = kUnitA + kUnitB;                // 9216
constexpr int kUnits = 8;                                  // gathered ring stages
constexpr int kAhead = kUnits - 1;                         // units in flight ahead
constexpr int kBatch = 64;                                 // units whose ids are staged
constexpr int kDataBytes = kStages * kStageDense;          // 73728
static_assert(kUnits * kUnitBytes == kDataBytes, "the two rings share one region");
constexpr int kOffEnt = kDataBytes;                        // uint16 [kBatch][32] channel ids
constexpr int kOffBp = kOffEnt + kBatch * KS * 2;          // uint64 [4][16] bound parts
constexpr int kOffOff = kOffBp + 4 * kTags * 8;            // int32 [4][65] bin offsets
constexpr int kOffRs = kOffOff + 4 * (kBins + 1) * 4;      // int32 [4][16] prefix starts
constexpr int kOffRc = kOffRs + 4 * kTags * 4;             // int32 [4][16] prefix lengths
constexpr int kOffUs = kOffRc + 4 * kTags * 4;             // int32 [65] (+pad) unit starts
constexpr int kOffUi = kOffUs + 68 * 4;                    // uint32 [kBatch] unit tile/rows
constexpr int kOffElig = kOffUi + kBatch * 4;              // int32 [4]
constexpr int kLdsBytes = kOffElig + 4 * 4;
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
constexpr int kWaitVmChunk = wait_vm(6);   // one dense chunk's six loads
constexpr int kWaitVmChunkIds = wait_vm(14);  // ... and eight id loads
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

// The same from a gathered W tile [32 channels][256 columns] whose 16-byte
// pieces are stored XOR-swizzled: column piece P of channel c sits at piece
// P ^ (c mod 8), so the 8 channels one 16-lane group reads hit 8 different
// pieces (no bank conflicts).  Channels c and c + 8 share the swizzle.
__device__ __forceinline__ v4i tr_frag_wsw(const uint8_t* tile, int col0, int lane) {
  const int q = lane >> 4, r = lane & 15;
  const int c = 16 * (q >> 1) + (r >> 1);
  const int piece = ((col0 >> 4) + (q & 1)) ^ (c & 7);
  const uint8_t* p = tile + c * BN + 16 * piece + 8 * (r & 1);
  const v2i lo = tr8(p);
  const v2i hi = tr8(p + 8 * BN);
  return v4i{lo[0], lo[1], hi[0], hi[1]};
}

__device__ __forceinline__ void shift_acc(v16i& acc, int s) {
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = (int)((uint32_t)acc[r] << s);
}

// Waits until at most `ops * after` vector-memory operations of this wave are
// in flight (after = 0 .. kAhead - 1).
template <int ops>
__device__ __forceinline__ void wait_units(int after) {
  switch (after) {
    case 0: __builtin_amdgcn_s_waitcnt(wait_vm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(wait_vm(ops * 1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(wait_vm(ops * 2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(wait_vm(ops * 3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(wait_vm(ops * 4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(wait_vm(ops * 5)); break;
    default: __builtin_amdgcn_s_waitcnt(wait_vm(ops * 6)); break;
  }
}

template <int T, bool VecW>
__global__ __launch_bounds__(kThreads, 2) void linear_mfma_kernel(LinearArgs a, int32_t row_blocks,
                                                                  int32_t col_blocks) {
  constexpr int kTiles = Cfg<T>::kTiles;
  // Direct-to-LDS loads per wave per gathered unit: one dword load of codes,
  // and the W rows as two 16-byte or eight 4-byte loads.
  constexpr int kOpsUnit = VecW ? 3 : 9;
  static_assert(kOpsUnit * (kAhead - 1) <= 63, "vmcnt range");
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* ent = reinterpret_cast<uint16_t*>(smem + kOffEnt);         // [kBatch][32]
  unsigned long long* bpart = reinterpret_cast<unsigned long long*>(smem + kOffBp);
  int32_t* off_s = reinterpret_cast<int32_t*>(smem + kOffOff);          // [kTiles][65]
  int32_t* rstart = reinterpret_cast<int32_t*>(smem + kOffRs);          // [kTiles][16]
  int32_t* rcount = reinterpret_cast<int32_t*>(smem + kOffRc);          // [kTiles][16]
  int32_t* ustart = reinterpret_cast<int32_t*>(smem + kOffUs);          // [65]
  uint32_t* uinfo = reinterpret_cast<uint32_t*>(smem + kOffUi);         // [kBatch]
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

  // ---- Dense ring: every channel with PoT ≤ 6, natural order, 64 channels
  // per chunk, filled by direct global-to-LDS loads (no registers): A = the
  // 128 rows of aligned codes, shared by the four waves; B = each wave's 64
  // columns of W^T.  Both tiles are [row][64 channels] with the 16-byte
  // columns XOR-swizzled by row, (column ^ (row / 4) % 4), so the fragment
  // reads (one ds_read_b128) are free of bank conflicts.  A direct load
  // writes lane l's 16 bytes at base + 16·l: one wave instruction fills 16
  // rows.  Each wave issues 2 A and 4 B instructions per chunk.
  auto stageA = [&](int st) { return smem + st * kStageDense; };
  auto stageB = [&](int st, int w) { return smem + st * kStageDense + BM * BK + w * WN * BK; };
  const int r16 = lane >> 2;                       // row of this lane within a 16-row group
  const int c16 = (lane & 3) ^ ((r16 >> 2) & 3);   // global 16-byte column it loads
  const int64_t nchunks = K / BK;
  auto issue = [&](int64_t c, int st) {
    const int64_t k0 = c * BK;
    const bool live = c < nchunks;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 16 * (2 * wave + j) + r16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_ac, (lds_ptr)(stageA(st) + 1024 * (2 * wave + j)), 16,
                                               live ? (uint32_t)(row * K + k0 + 16 * c16) : kOob, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = nw + 16 * j + r16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_wt, (lds_ptr)(stageB(st, wave) + 1024 * j), 16,
                                               live && n < N ? (uint32_t)(n * K + k0 + 16 * c16) : kOob, 0, 0, 0);
    }
  };

  // ---- Meta, overlapped with the first dense chunks: per tile and FPoT
  // group the prefix of the group (in perm) whose channels have PoT ≥ 7, the
  // exactness bound Σ_k 2^PoT_k, and the schedule of gathered units (32-row
  // block major, then group, then 32-channel step).
  // (Unconditional loads: the compiler then waits for exactly these, not for
  // the dense loads issued after them.)
  const rsrc_t r_off = make_rsrc(a.group_off + tile0 * (kBins + 1), (uint32_t)(tiles_here * (kBins + 1) * 4));
  uint32_t go[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int idx = tid + kThreads * m;
    go[m] = __builtin_amdgcn_raw_buffer_load_b32(r_off, idx < kTiles * (kBins + 1) ? (uint32_t)(4 * idx) : kOob, 0, 0);
  }
  __asm__ __volatile__("" ::: "memory");   // keep these loads ahead of the dense ones
#pragma unroll
  for (int c = 0; c < kStages - 1; ++c) issue(c, c);   // a chunk past K loads zeros
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int idx = tid + kThreads * m;
    if (idx < kTiles * (kBins + 1)) off_s[idx] = (int32_t)go[m];
  }
  bar_lds();
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
  bar_lds();
  if (wave == 0) {
    // lane = 16 · (32-row block) + group
    const int rb = lane >> 4, g = lane & 15, i = (32 * rb) / T;
    unsigned long long b = 0;
    for (int g2 = 0; g2 < kTags; ++g2) b += bpart[i * kTags + g2];
    const bool el = i < tiles_here && b <= kBoundLimit;
    if (g == 0 && (32 * rb) % T == 0) eligible[i] = el ? 1 : 0;
    int v = el ? (rcount[i * kTags + g] + KS - 1) / KS : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(v, o, 64);
      if (lane >= o) v += n;
    }
    ustart[lane + 1] = v;
    if (lane == 0) ustart[0] = 0;
  }
  bar_lds();
  const int U = ustart[RB * kTags];   // gathered units of this workgroup

  // Channel ids of units [ubase, ubase + kBatch): thread → (unit, 8 ids).
  // fetch() issues the loads into registers, commit() writes them to LDS.
  uint32_t fid[8], fok, finfo;
  auto fetch = [&](int ubase) {
    const int uu = ubase + (tid >> 2), qq = tid & 3;
    int lo = 0;
#pragma unroll
    for (int st = 32; st >= 1; st >>= 1)   // largest x with ustart[x] <= uu
      if (lo + st < RB * kTags && ustart[lo + st] <= uu) lo += st;
    const bool valid = uu < U;
    const int rb = lo >> 4, g = lo & 15, i = (32 * rb) / T;
    const int s = uu - ustart[lo];
    const int cnt = valid ? rcount[i * kTags + g] : 0;
    const int64_t base = (int64_t)i * K + rstart[i * kTags + g];
    // (The loaded ids are only touched in commit(), so the loads stay in
    // flight until then.)
    fok = 0;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int pos = KS * s + 8 * qq + jj;
      const bool ok = pos < cnt;
      fid[jj] = __builtin_amdgcn_raw_buffer_load_b16(r_perm, ok ? (uint32_t)((base + pos) * 2) : kOob, 0, 0);
      fok |= (ok ? 1u : 0u) << jj;
    }
    finfo = (uint32_t)i | ((uint32_t)(rb % (T / 32)) << 2);
  };
  auto commit = [&]() {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) fid[jj] = ((fok >> jj) & 1u) ? (fid[jj] & 0xFFFFu) : 0xFFFFu;
    uint4 p;
    p.x = fid[0] | (fid[1] << 16);
    p.y = fid[2] | (fid[3] << 16);
    p.z = fid[4] | (fid[5] << 16);
    p.w = fid[6] | (fid[7] << 16);
    *reinterpret_cast<uint4*>(ent + (tid >> 2) * KS + 8 * (tid & 3)) = p;
    if ((tid & 3) == 0) uinfo[tid >> 2] = finfo;
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

  // ---- Dense loop.
  {
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
    for (int64_t c = 0; c < nchunks; ++c) {
      // Chunk c's loads are done once at most one later chunk is in flight.
      // The barrier then makes every wave's part of chunk c visible and
      // guarantees every wave is done with chunk c - 1 (whose stage the next
      // loads overwrite).
      // (In the first two iterations the eight id loads issued after chunk 1
      // may also be in flight.)
      if (c + 1 >= nchunks) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      } else if (c < 2) {
        __builtin_amdgcn_s_waitcnt(kWaitVmChunkIds);
      } else {
        __builtin_amdgcn_s_waitcnt(kWaitVmChunk);
      }
      __asm__ __volatile__("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ __volatile__("" ::: "memory");
      if (c + kStages - 1 < nchunks) issue(c + kStages - 1, (int)((c + kStages - 1) % kStages));
      compute((int)(c % kStages));
    }
  }

  // ---- Epilogue set-up.  Y is streamed once: its loads and stores are
  // non-temporal so they do not evict W and the codes from the caches.  In
  // interior blocks the epilogue runs over (32-row block, 32-column block)
  // units, loading the next unit's Y_{t−1} before storing the current one;
  // the first unit's loads are issued here, under the gathered phase.
  // Offsets are 32-bit, relative to this workgroup's first row.
  const double base = a.base;
  bool all_eligible = true;
#pragma unroll
  for (int i = 0; i < kTiles; ++i) all_eligible = all_eligible && eligible[i];
  const bool interior = all_eligible && (tile0 * T + BM <= a.rows) && (nw + WN <= N);
  constexpr int kNt = 2;   // aux bit: non-temporal
  const rsrc_t r_yp = make_rsrc(a.y_prev + tile0 * T * N, (uint32_t)(BM * N * 4));
  const rsrc_t r_yo = make_rsrc(a.y_out + tile0 * T * N, (uint32_t)(BM * N * 4));
  const uint32_t lane_off = (uint32_t)(((4 * h) * N + nw + li) * 4);
  const uint32_t row4 = (uint32_t)(N * 4);
  auto y_off = [&](int rb, int cb, int r) {
    return lane_off + (uint32_t)(32 * rb + 8 * (r >> 2) + (r & 3)) * row4 + 128 * cb;
  };
  float ypa[16], ypb[16];
  auto load_y = [&](float (&dst)[16], int rb, int cb) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      dst[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_yp, y_off(rb, cb, r), 0, kNt));
  };
  if (interior) load_y(ypa, 0, 0);

  // ---- Gathered FPoT groups (channels with PoT ≥ 7), per 32-row block.
  // Unit v occupies ring stage v % kUnits: A = [32 channels][32 rows] codes,
  // B = [32 channels][256 columns] of W, swizzled.  Each wave loads 256 bytes
  // of A (dword loads: channel 8·wave + lane/8, dword lane % 8) and a quarter
  // of B.  Columns past N only feed outputs that are never stored.
  if (U > 0) {
    commit();
    bar_lds();   // ids visible; every wave is done with the dense ring
    int ubase = 0, u = 0, issued = 0;
    // Unit starts: lane x holds ustart[x] (x < 64), read with readlane.
    const int us_lane = ustart[lane];
    auto us_at = [&](int x) -> int { return x >= RB * kTags ? U : __builtin_amdgcn_readlane(us_lane, x); };
    // The ids one wave needs for one unit's loads (all LDS reads first, so
    // they share one wait).
    constexpr int kNB = VecW ? 2 : 8;
    struct UnitIds {
      uint32_t inf, chA, chB[kNB];
    };
    auto load_ids = [&](int v, UnitIds& d) {
      const uint16_t* en = ent + (v - ubase) * KS;
      d.inf = uinfo[v - ubase];
      d.chA = en[8 * wave + (lane >> 3)];
#pragma unroll
      for (int m = 0; m < kNB; ++m)
        d.chB[m] = VecW ? en[4 * (2 * wave + m) + (lane >> 4)] : en[8 * wave + m];
    };
    auto issue_ids = [&](int v, const UnitIds& d) {
      const int i = (int)(d.inf & 3u);
      const int rowoff = 32 * (int)(d.inf >> 2);
      uint8_t* sA = smem + (v % kUnits) * kUnitBytes;
      uint8_t* sB = sA + kUnitA;
      {
        const uint32_t off =
            d.chA != 0xFFFFu ? (uint32_t)(((int64_t)i * K + d.chA) * T + rowoff + 4 * (lane & 7)) : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r_codes, (lds_ptr)(sA + 256 * wave), 4, off, 0, 0, 0);
      }
#pragma unroll
      for (int m = 0; m < kNB; ++m) {
        const uint32_t ch = d.chB[m];
        if constexpr (VecW) {
          const int jj = 2 * wave + m;            // channels 4·jj .. 4·jj + 3
          const int c = 4 * jj + (lane >> 4);
          const int piece = (lane & 15) ^ (c & 7);
          const uint32_t off = ch != 0xFFFFu ? (uint32_t)((int64_t)ch * N + n0 + 16 * piece) : kOob;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r_w, (lds_ptr)(sB + 1024 * jj), 16, off, 0, 0, 0);
        } else {
          const int c = 8 * wave + m;             // one channel row of 256 bytes
          const int piece = (lane >> 2) ^ (c & 7);
          const uint32_t off =
              ch != 0xFFFFu ? (uint32_t)((int64_t)ch * N + n0 + 16 * piece + 4 * (lane & 3)) : kOob;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r_w, (lds_ptr)(sB + BN * c), 4, off, 0, 0, 0);
        }
      }
    };
    auto issue_unit = [&](int v) {
      UnitIds d;
      load_ids(v, d);
      issue_ids(v, d);
    };
    auto issue_upto = [&](int lim) {
      for (; issued < lim; ++issued) issue_unit(issued);
    };
    issue_upto(min(U, min(ubase + kBatch, kAhead)));
    // One gathered unit: wait for its loads, barrier, refill the ring, MFMA.
    auto step = [&](v16i (&tmp)[CB]) {
      if (u == ubase + kBatch) {
        bar_lds();   // every wave is done with the previous ids (no loads in flight)
        ubase = u;
        fetch(ubase);
        commit();
        bar_lds();
        issue_upto(min(U, min(ubase + kBatch, u + kAhead)));
      }
      const int hi = min(U, ubase + kBatch);
      // The next unit's ids are read before the wait (their stage is only
      // written after the barrier).
      const bool more = issued < min(hi, u + kAhead + 1);
      UnitIds nx;
      if (more) load_ids(issued, nx);
      wait_units<kOpsUnit>(min(kAhead - 1, hi - 1 - u));
      __asm__ __volatile__("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ __volatile__("" ::: "memory");
      if (more) {
        issue_ids(issued, nx);
        ++issued;
      }
      const uint8_t* sA = smem + (u % kUnits) * kUnitBytes;
      v4i af = tr_frag<32>(sA, 0, lane);
      v4i bf0 = tr_frag_wsw(sA + kUnitA, WN * wave, lane);
      v4i bf1 = tr_frag_wsw(sA + kUnitA, WN * wave + 32, lane);
      lgkm_wait(af, bf0, bf1);
      tmp[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf0, tmp[0], 0, 0, 0);
      tmp[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf1, tmp[1], 0, 0, 0);
      ++u;
    };
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (us_at((rb + 1) * kTags) == us_at(rb * kTags)) continue;
      v16i tmp[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmp[cb][r] = 0;
      int prev_e = -1;
      for (int g = 0; g < kTags; ++g) {
        const int nst = us_at(rb * kTags + g + 1) - us_at(rb * kTags + g);
        if (nst == 0) continue;
        const int e = DSTAR_FMDQ_TAG_OFFSET - g;
        if (prev_e >= 0) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) shift_acc(tmp[cb], prev_e - e);
        }
        prev_e = e;
        for (int s = 0; s < nst; ++s) step(tmp);
      }
      // Bring the gathered groups to units of the base and add them.
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[rb][cb][r] = (int)((uint32_t)acc[rb][cb][r] + ((uint32_t)tmp[cb][r] << prev_e));
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
#pragma unroll
    for (int v = 0; v < RB * CB; ++v) {
      const int rb = v / CB, cb = v % CB;
      float (&cur)[16] = (v & 1) ? ypb : ypa;
      float (&nxt)[16] = (v & 1) ? ypa : ypb;
      if (v + 1 < RB * CB) load_y(nxt, (v + 1) / CB, (v + 1) % CB);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const double d = __dmul_rn(__dmul_rn((double)acc[rb][cb][r], base), ws[cb]);
        const float y = (float)__dadd_rn((double)cur[r], d);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, y), r_yo, y_off(rb, cb, r), 0, kNt);
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
