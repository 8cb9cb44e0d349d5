// Stage 2 of the FMDQ differential linear: reorder the channels of each token
// tile by FPoT tag (DSTAR, arXiv 2607.15846: §3.1 step 3; §4.2 QPU stage 4).
//
// One workgroup per token tile runs an LDS counting sort.  Thread j owns the
// contiguous channel range [j*per, (j+1)*per).  It counts its tags into column
// j of a [16][256] LDS table; one exclusive scan over that table, read in
// row-major order, gives every (tag, thread) pair its first output slot, which
// is exactly the stable order (tag ascending, channel ascending).  The threads
// then place their channels in order.  For K <= 32768 the tags and the sorted
// ids are staged in LDS and moved with coalesced 16-byte accesses.
#include "fmdq_internal.h"

namespace dstar {
namespace {

constexpr int kThreads = 256;
constexpr int kTags = DSTAR_FMDQ_NUM_TAGS;
constexpr int kLdsMaxK = 32768;

// Exclusive scan of the 16*256 counters in `tab` (row-major [tag][thread]).
__device__ void exclusive_scan_table(uint32_t* tab, uint32_t* wave_tot) {
  const int tid = threadIdx.x;
  uint32_t v[16];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = tab[16 * tid + i];
    sum += v[i];
  }
  // inclusive scan of `sum` across the wave
  const int lane = tid & 63;
  uint32_t inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) wave_tot[tid >> 6] = inc;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < (tid >> 6); ++w) base += wave_tot[w];
  uint32_t run = base + inc - sum;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    tab[16 * tid + i] = run;
    run += v[i];
  }
  __syncthreads();
}

template <bool kInLds>
__global__ __launch_bounds__(kThreads) void bucket_kernel(BucketArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* tab = reinterpret_cast<uint32_t*>(smem);                    // [16][256]
  uint32_t* wave_tot = tab + kTags * kThreads;                          // [4]
  uint8_t* tags_s = smem + (kTags * kThreads + 16) * 4;                 // [K] (kInLds)
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
    for (int g = 0; g < kTags; ++g) tab[g * kThreads + tid] = 0u;
    if constexpr (kInLds) {
      for (int i = tid; i < K; i += kThreads) tags_s[i] = tg[i];
    }
    __syncthreads();
    const uint8_t* src = kInLds ? tags_s : tg;
    for (int k = kbeg; k < kend; ++k) tab[(src[k] & 15) * kThreads + tid] += 1u;
    __syncthreads();
    exclusive_scan_table(tab, wave_tot);
    if (tid < kTags) a.group_off[tile * (kTags + 1) + tid] = (int32_t)tab[tid * kThreads];
    if (tid == kTags) a.group_off[tile * (kTags + 1) + kTags] = K;
    __syncthreads();  // column 0 of the table is read above and updated below
    for (int k = kbeg; k < kend; ++k) {
      const int g = src[k] & 15;
      const uint32_t pos = tab[g * kThreads + tid];
      tab[g * kThreads + tid] = pos + 1u;
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
  const size_t base = (size_t)(kTags * kThreads + 16) * 4;
  if (a.K <= kLdsMaxK) {
    const size_t kpad = (size_t)((a.K + 15) & ~15);
    const size_t lds = base + kpad + 2 * kpad;
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)bucket_kernel<true>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess)
        return set_error(DSTAR_EHIP, "fmdq_bucket: hipFuncSetAttribute: %s", hipGetErrorString(e));
    }
    hipLaunchKernelGGL(bucket_kernel<true>, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  } else {
    hipLaunchKernelGGL(bucket_kernel<false>, dim3((unsigned)grid), dim3(kThreads), base, s, a);
  }
  return check_launch("fmdq_bucket");
}

}  // namespace dstar
