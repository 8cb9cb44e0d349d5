// Dynamic base of the FMDQ differential linear: the first of the two passes
// over X that a base taken from the data needs (DSTAR, arXiv 2607.15846: §3.1
// step 1 defines the base of Eq. 2-3 as the smallest sub-channel maximum M_i;
// the static base of the method removes this pass, and §5.2 Table 2 evaluates
// the dynamic variant as DS-FMDQ-DYN).
//
// base = min over sub-channels (token tile × channel) with M > 0 of
// M = max |X_t − X_{t−1}| over the tile's rows, clamped to [2^-100, 2^100];
// the static base when every M is 0.  M and its minimum are exact in float32,
// and a positive float32 orders like its bit pattern, so the minimum is an
// atomicMin over 32-bit patterns: one kernel writes +inf, the reduction
// lowers it (one atomic per wave), a last one-thread kernel applies the
// fallback and the clamp.  No memset, so the sequence can be captured in a
// HIP graph.
#include "fmdq_internal.h"

namespace dstar {
namespace {

constexpr int kThreads = 256;
typedef float f4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kInfBits = 0x7F800000u;

__global__ void base_init_kernel(uint32_t* bits) {
  if (threadIdx.x == 0) *bits = kInfBits;
}

// Workgroup = one token tile × 64·V channels; lane l of every wave owns
// channels [V·(64·slab + l), +V) (float4 loads when V = 4: K % 4 == 0 and
// 16-byte aligned rows), and wave w the rows [w·T/4, (w+1)·T/4) of the tile.
// The four partial maxima meet in LDS; wave 0 forms M and the minimum.  The
// RW = T/4 row loads of a lane are unconditional (a row past the end reads the
// last row and is ignored), so they are all in flight together.
//
// Workgroups stride over the (tile, slab) items and keep their minimum in a
// register; wave 0 then lowers the global value once, and only when its own
// minimum is below what it reads there (the stored value only decreases, so
// a stale read costs at most a needless atomic): atomics on one address
// are serialized, so their number is kept small.
template <int V, int RW>
__global__ __launch_bounds__(kThreads) void base_min_kernel(BaseArgs a, int32_t slabs, int64_t items) {
  __shared__ float part[kThreads / 64][64 * V];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t K = a.K;
  uint32_t best = kInfBits;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t tile = item / slabs;
    const int64_t slab = item - tile * slabs;
    const int64_t k = (slab * 64 + lane) * V;
    const int64_t r0 = tile * (int64_t)(4 * RW) + (int64_t)wave * RW;
    float m[V];
#pragma unroll
    for (int c = 0; c < V; ++c) m[c] = 0.0f;
    if (k < K) {
#pragma unroll
      for (int t = 0; t < RW; ++t) {
        const int64_t r = min(r0 + t, a.rows - 1);
        const bool live = r0 + t < a.rows;
        float xt[V], xp[V];
        if constexpr (V == 4) {
          const f4 u = __builtin_nontemporal_load(reinterpret_cast<const f4*>(a.x_t + r * K + k));
          const f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4*>(a.x_prev + r * K + k));
          xt[0] = u.x; xt[1] = u.y; xt[2] = u.z; xt[3] = u.w;
          xp[0] = v.x; xp[1] = v.y; xp[2] = v.z; xp[3] = v.w;
        } else {
          xt[0] = __builtin_nontemporal_load(a.x_t + r * K + k);
          xp[0] = __builtin_nontemporal_load(a.x_prev + r * K + k);
        }
#pragma unroll
        for (int c = 0; c < V; ++c) m[c] = fmaxf(m[c], live ? fabsf(__fsub_rn(xt[c], xp[c])) : 0.0f);
      }
    }
#pragma unroll
    for (int c = 0; c < V; ++c) part[wave][lane * V + c] = m[c];
    __syncthreads();
    if (wave == 0 && k < K) {
#pragma unroll
      for (int c = 0; c < V; ++c) {
        float mc = part[0][lane * V + c];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) mc = fmaxf(mc, part[w][lane * V + c]);
        if (mc > 0.0f) best = min(best, __float_as_uint(mc));
      }
    }
    __syncthreads();   // part is rewritten by the next item
  }
  if (wave != 0) return;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) best = min(best, (uint32_t)__shfl_xor((int)best, o, 64));
  if (lane == 0 && best != kInfBits) {
    const uint32_t cur = *reinterpret_cast<volatile const uint32_t*>(a.base_bits);
    if (best < cur) atomicMin(a.base_bits, best);
  }
}

__global__ void base_final_kernel(uint32_t* bits, float fallback) {
  if (threadIdx.x != 0) return;
  const uint32_t b = *bits;
  const float v = b == kInfBits ? fallback : fminf(fmaxf(__uint_as_float(b), 0x1p-100f), 0x1p100f);
  *reinterpret_cast<float*>(bits) = v;
}

template <int V, int RW>
int launch_v(const BaseArgs& a, hipStream_t s) {
  const int32_t slabs = (int32_t)((a.K + 64 * V - 1) / (64 * V));
  const int64_t items = n_tiles(a.rows, a.T) * slabs;
  const int64_t grid = items < 1024 ? items : 1024;
  hipLaunchKernelGGL((base_min_kernel<V, RW>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, slabs, items);
  return check_launch("fmdq_dynamic_base (min)");
}

template <int V>
int launch_t(const BaseArgs& a, hipStream_t s) {
  switch (a.T) {
    case 16: return launch_v<V, 4>(a, s);
    case 32: return launch_v<V, 8>(a, s);
    case 64: return launch_v<V, 16>(a, s);
    default: return set_error(DSTAR_EUNSUPPORTED, "dynamic_base: token_tile %d not supported", a.T);
  }
}

}  // namespace

int launch_dynamic_base(const BaseArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(base_init_kernel, dim3(1), dim3(64), 0, s, a.base_bits);
  if (int rc = check_launch("fmdq_dynamic_base (init)")) return rc;
  if (a.rows > 0) {
    const int rc = (a.K % 4) == 0 ? launch_t<4>(a, s) : launch_t<1>(a, s);
    if (rc) return rc;
  }
  hipLaunchKernelGGL(base_final_kernel, dim3(1), dim3(64), 0, s, a.base_bits, a.fallback);
  return check_launch("fmdq_dynamic_base (final)");
}

}  // namespace dstar
