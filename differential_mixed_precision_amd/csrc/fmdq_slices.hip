// The 2-bit slice stream of DSTAR's accelerator (arXiv 2607.15846: §3.1 step
// 2 sub-channel decomposition, step 3 reordering, step 4 encoding; §4.2 QPU
// stages 3-4), produced for inspection and for a 2-bit datapath.  The MFMA
// path of this library multiplies whole 8-bit codes and does not read it.
//
// A b-bit code is split into b/2 slices of 2 bits (the radix-4 digits of its
// two's-complement form; slice n is the field (q >> 2n) & 3, the top one read
// as signed), and slice n of a sub-channel takes the FPoT lowered by 2n, i.e.
// slice tag tag − 2n in [−6, 15], bin = slice tag + 6.  Per token tile the
// entries (channel, slice) are ordered by bin, then channel, and each carries
// the number of left shifts to apply to the running partial sum before it
// (the bin difference to the previous entry).
//
// One workgroup per token tile.  For each bin a bitmap over the channels
// marks the channels with an entry in that bin (LDS atomicOr); one exclusive
// scan over the popcounts of the bitmap words, in (bin, word) order, gives
// every word its first slot, and an entry's slot is that plus the number of
// lower set bits in its word — the (bin, channel) order without a sort.
#include "fmdq_internal.h"

namespace dstar {
namespace {

constexpr int kThreads = 256;
constexpr int kSliceBins = 22;
constexpr int kSliceTagOff = 6;

__global__ __launch_bounds__(kThreads) void slice_kernel(SliceArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = a.K, T = a.T;
  const int W = (K + 31) / 32;                                          // bitmap words per bin
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem);                     // [22][W]
  int32_t* offs = reinterpret_cast<int32_t*>(smem + 4 * kSliceBins * W);  // [22][W] (+1 total)
  int32_t* prevb = offs + kSliceBins * W + 1;                           // [22]
  uint32_t* wave_tot = reinterpret_cast<uint32_t*>(prevb + kSliceBins);  // [4]
  uint8_t* tags_s = reinterpret_cast<uint8_t*>(wave_tot + 4);           // [K]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = kSliceBins * W;
  const int per = (E + kThreads - 1) / kThreads;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);

  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    const uint8_t* tg = a.tags + tile * (int64_t)K;
    for (int i = tid; i < K; i += kThreads) tags_s[i] = tg[i];
    for (int i = tid; i < E; i += kThreads) bm[i] = 0u;
    __syncthreads();
    for (int k = tid; k < K; k += kThreads) {
      const uint32_t t = tags_s[k];
      const int g = (int)(t & 15u), nsl = (int)((t >> DSTAR_FMDQ_PREC_SHIFT) & 3u) + 1;
      for (int n = 0; n < nsl; ++n)
        atomicOr(&bm[(g - 2 * n + kSliceTagOff) * W + (k >> 5)], 1u << (k & 31));
    }
    __syncthreads();
    // exclusive scan of the word popcounts in (bin, word) order
    uint32_t sum = 0;
    for (int e = e0; e < e1; ++e) sum += __popc(bm[e]);
    uint32_t inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    uint32_t run = inc - sum;
    for (int w = 0; w < wave; ++w) run += wave_tot[w];
    for (int e = e0; e < e1; ++e) {
      offs[e] = (int32_t)run;
      run += __popc(bm[e]);
    }
    if (tid == kThreads - 1) offs[E] = (int32_t)run;   // the last thread's run is the total
    __syncthreads();
    if (tid < kSliceBins) {
      int p = -1;
      for (int b = tid - 1; b >= 0; --b) {
        if (offs[(b + 1) * W] > offs[b * W]) { p = b; break; }
      }
      prevb[tid] = p;
    }
    if (tid <= kSliceBins)
      a.slice_off[tile * (kSliceBins + 1) + tid] = tid < kSliceBins ? offs[tid * W] : offs[E];
    __syncthreads();
    const int8_t* cd = a.codes + tile * (int64_t)K * T;
    uint32_t* ent = a.entries + tile * 4 * (int64_t)K;
    uint8_t* dat = a.slices + tile * 4 * (int64_t)K * (T / 4);
    const int total = offs[E];
    for (int k = tid; k < K; k += kThreads) {
      const uint32_t t = tags_s[k];
      const int g = (int)(t & 15u), nsl = (int)((t >> DSTAR_FMDQ_PREC_SHIFT) & 3u) + 1;
      // the code's T bytes, as 32-bit words
      uint32_t cw[16];
#pragma unroll
      for (int v = 0; v < 16; ++v)
        cw[v] = v < T / 4 ? *reinterpret_cast<const uint32_t*>(cd + (int64_t)k * T + 4 * v) : 0u;
      for (int n = 0; n < nsl; ++n) {
        const int b = g - 2 * n + kSliceTagOff;
        const uint32_t word = bm[b * W + (k >> 5)];
        const int pos = offs[b * W + (k >> 5)] + __popc(word & ((1u << (k & 31)) - 1u));
        const bool first = pos == offs[b * W];
        const int shift = (first && prevb[b] >= 0) ? b - prevb[b] : 0;
        ent[pos] = (uint32_t)k | ((uint32_t)n << 16) | ((uint32_t)shift << 24);
        // rows 4v .. 4v+3 of word v -> one byte of 2-bit fields
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if (v < T / 4) {
            const uint32_t x = cw[v];
            uint32_t byte = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) byte |= (((x >> (8 * i)) >> (2 * n)) & 3u) << (2 * i);
            dat[(int64_t)pos * (T / 4) + v] = (uint8_t)byte;
          }
        }
      }
    }
    // entries past the tile's count
    for (int j = total + tid; j < 4 * K; j += kThreads) ent[j] = 0xFFFFFFFFu;
    __syncthreads();
  }
}

}  // namespace

int launch_slices(const SliceArgs& a, hipStream_t s) {
  if (a.n_tiles == 0) return DSTAR_OK;
  const int64_t grid = a.n_tiles < 2048 ? a.n_tiles : 2048;
  const size_t W = (size_t)((a.K + 31) / 32);
  const size_t lds = 4 * kSliceBins * W + 4 * (kSliceBins * W + 1) + 4 * kSliceBins + 16 + (size_t)a.K;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)slice_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess)
      return set_error(DSTAR_EHIP, "fmdq_slice_encode: hipFuncSetAttribute: %s", hipGetErrorString(e));
  }
  hipLaunchKernelGGL(slice_kernel, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  return check_launch("fmdq_slice_encode");
}

}  // namespace dstar
