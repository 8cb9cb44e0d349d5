// Stage 2 of the FMDQ differential linear: reorder the channels of each token
// tile by FPoT tag (DSTAR, arXiv 2607.15846: §3.1 step 3; §4.2 QPU stage 4).
//
// Order: FPoT tag ascending; inside one tag, precision descending; then
// channel ascending.  The key of a channel is bin = 4·tag + (3 − precision
// code), 64 bins.  (The pages fix only the FPoT order; the precision order
// makes the sub-channels whose shift-aligned codes need more than 8 bits a
// prefix of every FPoT group, which the GEMM of stage 3 reads directly.)
//
// One workgroup per token tile runs an LDS counting sort.  Thread j owns the
// contiguous channel range [j*per, (j+1)*per).  It counts its keys into column
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
