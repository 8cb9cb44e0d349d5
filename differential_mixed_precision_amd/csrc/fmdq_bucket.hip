// Stage 2 of the FMDQ differential linear: reorder the channels of each token
// tile by FPoT tag (DSTAR, arXiv 2607.15846: §3.1 step 3; §4.2 QPU stage 4).
//
// Order: FPoT tag ascending; inside one tag, precision descending; then
// channel ascending.  The key of a channel is bin = 4·tag + (3 − precision
// code), 64 bins.  (The pages fix only the FPoT order; the precision order
// makes the sub-channels whose shift-aligned codes need more than 8 bits a
// prefix of every FPoT group, which the GEMM of stage 3 reads directly.)
//
// One workgroup per token tile runs an LDS counting sort.
//
// For K <= 16384 (every workload) the count is a wave-level split: a wave
// takes 64 consecutive channels ("chunk"), and for each lane the lanes with
// the same bin come from a per-wave LDS table of 64 lane masks (each lane ORs
// its bit into its bin's entry and reads the entry back); the lowest of them
// writes the group's size into a [64 bins][chunks] table, and a lane's rank
// among its peers is the number of lower peers.  Each lane keeps its bin and
// rank in a register from the count to the placement, and a wave loads the
// tags of all its chunks (16 at most) at once, straight from global memory.
// One exclusive scan over the table in (bin, chunk) order then gives every
// (bin, chunk) its first output slot — the stable order, since chunks and
// lanes both run in channel order — and each lane places its channel at
// slot + rank.  No step is a chain of dependent LDS updates.
//
// Otherwise thread j owns the contiguous channel range [j*per, (j+1)*per).  It counts its keys into column
// j of a [64][256] uint16 LDS table; one exclusive scan over that table, read
// in row-major order, gives every (bin, thread) pair its first output slot,
// which is exactly the stable order.  The threads then place their channels
// in order.  For K <= 32768 the tags and the sorted ids are staged in LDS and
// moved with coalesced accesses.
#include "fmdq_internal.h"

namespace dstar {
namespace {

constexpr int kThreads = 256;
constexpr int kBins = DSTAR_FMDQ_NUM_BINS;
constexpr int kLdsMaxK = 32768;
constexpr int kPerScan = kBins * kThreads / kThreads;  // table entries scanned per thread (64)

__device__ __forceinline__ int bin_of(uint32_t tag_byte) {
  return 4 * (int)(tag_byte & 15u) + (3 - (int)((tag_byte >> DSTAR_FMDQ_PREC_SHIFT) & 3u));
}

// Exclusive scan, in place, of the 64*256 uint16 counters of `tab` taken in
// row-major order ([bin][thread]).  Every prefix is at most K <= 65535.
__device__ void exclusive_scan_table(uint16_t* tab, uint32_t* wave_tot) {
  const int tid = threadIdx.x;
  uint32_t* row = reinterpret_cast<uint32_t*>(tab + kPerScan * tid);  // 64 entries = 32 words
  uint32_t v[kPerScan / 2];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < kPerScan / 2; ++i) {
    v[i] = row[i];
    sum += (v[i] & 0xFFFFu) + (v[i] >> 16);
  }
  const int lane = tid & 63;
  uint32_t inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) wave_tot[tid >> 6] = inc;
  __syncthreads();
  uint32_t run = inc - sum;
  for (int w = 0; w < (tid >> 6); ++w) run += wave_tot[w];
#pragma unroll
  for (int i = 0; i < kPerScan / 2; ++i) {
    const uint32_t lo = run;
    run += v[i] & 0xFFFFu;
    const uint32_t hi = run;
    run += v[i] >> 16;
    row[i] = (lo & 0xFFFFu) | (hi << 16);
  }
  __syncthreads();
}

constexpr int kBallotMaxK = 16384;
constexpr int kBallotThreads = 1024;   // 16 waves: the chunks of one tile spread over them

// Row stride (uint16 entries) of the [64 bins][C chunks] count table: C
// rounded up so that a row spans an odd number of 4-byte words, which puts
// the entries of one chunk for different bins in different LDS banks (with C
// a multiple of 64, every bin of a chunk fell in the same bank).
__host__ __device__ __forceinline__ int count_row(int C) {
  const int w = (C + 1) / 2;
  return 2 * (w % 2 == 1 ? w : w + 1);
}

constexpr int kBallotWaves = kBallotThreads / 64;

// NCH bounds both the chunks of a wave (⌈C/16⌉) and the count-table entries
// a thread scans (⌈64·C/1024⌉, the same number); the host picks the smallest
// of 1, 2, 4, 8, 16 that covers K.
template <int NCH>
__global__ __launch_bounds__(kBallotThreads) void bucket_ballot_kernel(BucketArgs a) {
  constexpr int kChunksPerWave = NCH;
  constexpr int kScanPer = NCH;
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = a.K;
  const int C = (K + 63) / 64;                  // chunks of 64 channels
  const int E = kBins * C;                      // table entries, bin-major
  const int CP = count_row(C);                  // row stride of the table
  const int epad = (kBins * CP + 7) & ~7;
  uint16_t* cnt = reinterpret_cast<uint16_t*>(smem);                   // [64][CP]
  uint32_t* wave_tot = reinterpret_cast<uint32_t*>(smem + 2 * epad);   // [16]
  unsigned long long* mk = reinterpret_cast<unsigned long long*>(smem + 2 * epad + 64);   // [16 waves][64]
  uint16_t* perm_s = reinterpret_cast<uint16_t*>(smem + 2 * epad + 64 + 8 * kBallotThreads);  // [K]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  const unsigned long long me = 1ull << lane;
  mk += 64 * wave;
  const int per = (E + kBallotThreads - 1) / kBallotThreads;   // scan entries per thread (≤ NCH)
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  // Ids in 16-byte pieces when every tile's row is so aligned (the staging
  // buffer in LDS always is).
  const bool perm16 = ((reinterpret_cast<uintptr_t>(a.perm) | (uintptr_t)(2 * K)) & 15u) == 0;

  // one tile per workgroup (the grid is the tiles): nothing is carried from a
  // tile to the next, so nothing is held across one
  {
    const int64_t tile = blockIdx.x;
    const uint8_t* tg = a.tags + tile * (int64_t)K;
    uint16_t* out = a.perm + tile * (int64_t)K;
    // The wave's chunks are c = wave + 16·i.  Their tags are loaded at once
    // (clamped indices, so the number of loads is fixed and all are in
    // flight together) while the count table is cleared.
    uint32_t tb[kChunksPerWave];
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) tb[i] = tg[min(64 * (wave + kBallotWaves * i) + lane, K - 1)];
    for (int i = tid; i < epad / 8; i += kBallotThreads) reinterpret_cast<uint4*>(cnt)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    // Count.  A lane's bin and its rank among the lanes of its chunk with the
    // same bin stay in a register (bin | rank << 8) until the placement.
    // The lanes of a chunk with this lane's bin: every lane clears its own
    // entry of the wave's [64] mask table, ORs its lane bit into the entry of
    // its bin and reads that entry back.  A wave's LDS operations execute in
    // the order issued, so the three steps of a chunk (and the next chunk's
    // clear after this chunk's read) need no wait between them; the compiler
    // barriers keep that order in the code.
    uint64_t peers[kChunksPerWave];
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) {
      const int c = wave + kBallotWaves * i;
      peers[i] = 0;
      if (c < C) {                                 // wave-uniform
        const bool act = 64 * c + lane < K;
        const int bin = bin_of(tb[i]);
        mk[lane] = 0ull;
        __builtin_amdgcn_wave_barrier();
        if (act) atomicOr(&mk[bin], me);
        __builtin_amdgcn_wave_barrier();
        peers[i] = mk[bin];
        __builtin_amdgcn_wave_barrier();
      }
    }
    uint32_t br[(kChunksPerWave + 1) / 2];        // two (bin | rank << 8) halves per word
#pragma unroll
    for (int i = 0; i < (kChunksPerWave + 1) / 2; ++i) br[i] = 0;
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) {
      const int c = wave + kBallotWaves * i;
      if (c < C) {
        const bool act = 64 * c + lane < K;
        const int bin = bin_of(tb[i]);
        const uint32_t rank = (uint32_t)__popcll(peers[i] & below);
        if (act && rank == 0u) cnt[bin * CP + c] = (uint16_t)__popcll(peers[i]);
        br[i / 2] |= ((uint32_t)bin | (rank << 8)) << (16 * (i & 1));
      }
    }
    __syncthreads();
    // Exclusive scan of cnt in (bin, chunk) order: a thread's entries are
    // read at once, summed, offset by the wave scan and the lower waves'
    // totals, and written back from registers.
    uint32_t v[kScanPer];
    {
      int bb = e0 / max(C, 1), cc = e0 - bb * C;
#pragma unroll
      for (int i = 0; i < kScanPer; ++i) {
        v[i] = e0 + i < e1 ? cnt[bb * CP + cc] : 0u;
        if (++cc == C) { cc = 0; ++bb; }
      }
    }
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) sum += v[i];
    uint32_t inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t n = __shfl_up(inc, o, 64);
      if (lane >= o) inc += n;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    uint32_t run = inc - sum;
    for (int w = 0; w < wave; ++w) run += wave_tot[w];
    {
      int bb = e0 / max(C, 1), cc = e0 - bb * C;
#pragma unroll
      for (int i = 0; i < kScanPer; ++i) {
        if (e0 + i < e1) cnt[bb * CP + cc] = (uint16_t)run;
        run += v[i];
        if (++cc == C) { cc = 0; ++bb; }
      }
    }
    __syncthreads();
    if (tid < kBins) a.group_off[tile * (kBins + 1) + tid] = (int32_t)cnt[tid * CP];
    if (tid == kBins) a.group_off[tile * (kBins + 1) + kBins] = K;
    // Place: channel k goes to its (bin, chunk) slot plus its rank.
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) {
      const int c = wave + kBallotWaves * i;
      const int k = 64 * c + lane;
      const uint32_t v2 = (br[i / 2] >> (16 * (i & 1))) & 0xFFFFu;
      if (c < C && k < K) perm_s[cnt[(int)(v2 & 0xFFu) * CP + c] + (v2 >> 8)] = (uint16_t)k;
    }
    __syncthreads();
    if (perm16) {
      for (int i = tid; i < K / 8; i += kBallotThreads)
        reinterpret_cast<uint4*>(out)[i] = reinterpret_cast<const uint4*>(perm_s)[i];
    } else {
      for (int i = tid; i < K; i += kBallotThreads) out[i] = perm_s[i];
    }
  }
}

template <bool kInLds>
__global__ __launch_bounds__(kThreads) void bucket_kernel(BucketArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* tab = reinterpret_cast<uint16_t*>(smem);                   // [64][256]
  uint32_t* wave_tot = reinterpret_cast<uint32_t*>(smem + kBins * kThreads * 2);  // [4]
  uint8_t* tags_s = smem + kBins * kThreads * 2 + 64;                   // [K] (kInLds)
  const int K = a.K;
  const int kpad = (K + 15) & ~15;
  uint16_t* perm_s = reinterpret_cast<uint16_t*>(tags_s + kpad);       // [K] (kInLds)
  const int tid = threadIdx.x;
  const int per = (K + kThreads - 1) / kThreads;
  const int kbeg = min(K, tid * per);
  const int kend = min(K, kbeg + per);

  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    const uint8_t* tg = a.tags + tile * (int64_t)K;
    uint16_t* out = a.perm + tile * (int64_t)K;
#pragma unroll
    for (int b = 0; b < kBins; ++b) tab[b * kThreads + tid] = 0;
    if constexpr (kInLds) {
      for (int i = tid; i < K; i += kThreads) tags_s[i] = tg[i];
    }
    __syncthreads();
    const uint8_t* src = kInLds ? tags_s : tg;
    for (int k = kbeg; k < kend; ++k) tab[bin_of(src[k]) * kThreads + tid] += 1;
    __syncthreads();
    exclusive_scan_table(tab, wave_tot);
    if (tid < kBins) a.group_off[tile * (kBins + 1) + tid] = (int32_t)tab[tid * kThreads];
    if (tid == kBins) a.group_off[tile * (kBins + 1) + kBins] = K;
    __syncthreads();  // column 0 of the table is read above and updated below
    for (int k = kbeg; k < kend; ++k) {
      const int b = bin_of(src[k]);
      const uint32_t pos = tab[b * kThreads + tid];
      tab[b * kThreads + tid] = (uint16_t)(pos + 1u);
      if constexpr (kInLds) {
        perm_s[pos] = (uint16_t)k;
      } else {
        out[pos] = (uint16_t)k;
      }
    }
    if constexpr (kInLds) {
      __syncthreads();
      for (int i = tid; i < K; i += kThreads) out[i] = perm_s[i];
    }
    __syncthreads();
  }
}

}  // namespace

int launch_bucket(const BucketArgs& a, hipStream_t s) {
  if (a.n_tiles == 0) return DSTAR_OK;
  const int64_t grid = a.n_tiles < 2048 ? a.n_tiles : 2048;
  if (a.K <= kBallotMaxK) {
    const size_t E = (size_t)kBins * count_row((a.K + 63) / 64);
    const size_t lds = 2 * ((E + 7) & ~(size_t)7) + 64 + 8 * (size_t)kBallotThreads + 2 * (size_t)((a.K + 15) & ~15);
    if (lds > 65536) {
      // only the widest instantiation (K > 8192) needs more than 64 KB
      hipError_t e = hipFuncSetAttribute((const void*)bucket_ballot_kernel<16>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess)
        return set_error(DSTAR_EHIP, "fmdq_bucket: hipFuncSetAttribute: %s", hipGetErrorString(e));
    }
    // one workgroup per tile, at most 2^20 tiles (2^30 threads) per launch
    constexpr int64_t kMaxGrid = int64_t(1) << 20;
    for (int64_t t0 = 0; t0 < a.n_tiles; t0 += kMaxGrid) {
      BucketArgs b = a;
      b.n_tiles = a.n_tiles - t0 < kMaxGrid ? a.n_tiles - t0 : kMaxGrid;
      b.tags = a.tags + t0 * a.K;
      b.perm = a.perm + t0 * a.K;
      b.group_off = a.group_off + t0 * (kBins + 1);
      const int C = (a.K + 63) / 64;
      const dim3 grid((unsigned)b.n_tiles), block(kBallotThreads);
      if (C <= 16) hipLaunchKernelGGL(bucket_ballot_kernel<1>, grid, block, lds, s, b);
      else if (C <= 32) hipLaunchKernelGGL(bucket_ballot_kernel<2>, grid, block, lds, s, b);
      else if (C <= 64) hipLaunchKernelGGL(bucket_ballot_kernel<4>, grid, block, lds, s, b);
      else if (C <= 128) hipLaunchKernelGGL(bucket_ballot_kernel<8>, grid, block, lds, s, b);
      else hipLaunchKernelGGL(bucket_ballot_kernel<16>, grid, block, lds, s, b);
      if (int rc = check_launch("fmdq_bucket")) return rc;
    }
    return DSTAR_OK;
  }
  const size_t base = (size_t)kBins * kThreads * 2 + 64;
  size_t lds = base;
  const void* fn = (const void*)bucket_kernel<false>;
  if (a.K <= kLdsMaxK) {
    const size_t kpad = (size_t)((a.K + 15) & ~15);
    lds = base + kpad + 2 * kpad;
    fn = (const void*)bucket_kernel<true>;
  }
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
      return set_error(DSTAR_EHIP, "fmdq_bucket: hipFuncSetAttribute: %s", hipGetErrorString(e));
  }
  if (a.K <= kLdsMaxK) {
    hipLaunchKernelGGL(bucket_kernel<true>, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  } else {
    hipLaunchKernelGGL(bucket_kernel<false>, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  }
  return check_launch("fmdq_bucket");
}

}  // namespace dstar
