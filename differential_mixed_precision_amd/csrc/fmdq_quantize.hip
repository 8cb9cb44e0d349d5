// Stage 1 of the FMDQ differential linear: fused differential + sub-channel
// quantization (DSTAR, arXiv 2607.15846: §2.2 Eq. 1; §3.1 step 1 with Eq. 2-5;
// §4.2 QPU stages 1-3).
//
// HBM-bound streaming kernel.  A group of G = T/16 adjacent lanes (one lane
// at T = 16; T/8 for the small launches at T = 32, see launch_quantize) owns
// CPT adjacent input channels of one token tile; each lane of the group reads
// 16 (or 8) of the tile's T rows of X_t and X_{t-1} for those
// channels with CPT-wide vector loads (non-temporal: X is read once), keeps
// its Δ in registers and reduces max|Δ| per channel; shuffles within the
// group give the sub-channel maximum M.  Every lane then picks PoT /
// precision / tag with exact float32 compares against base*2^j and quantizes
// its rows.  Each lane writes its rows of a channel's T codes (codes are
// channel-major within a tile: a contiguous run per lane), its rows of the
// aligned codes (one CPT-byte word per row), and the group's first lane
// writes the tags and counts the bit histogram.  A code in units
// of the base, a = q·2^e, is the aligned code itself when PoT ≤ 6; otherwise
// it is split into signed digits a = d0 + 2^7·d1 + 2^15·d2: d0 goes to the
// aligned codes, d1 (PoT ≥ 7) and d2 (PoT ≥ 14) to the two digit planes, laid
// out like the codes.
#include "fmdq_internal.h"

namespace dstar {
namespace {

constexpr int kThreads = 256;
constexpr int RT = 16;                  // rows per lane
// Workgroups of a launch: the ones resident at once (two per CU at two waves
// per SIMD, 256 CUs), each striding over the work items.  Measured on the
// PixArt-alpha step: fc1 29 -> 26 us and fc2 74 -> 72 us against one
// workgroup per item; 256, 384, 640 ... 2048 were all slower.
constexpr int64_t kMaxGrid = 512;

typedef float fv4 __attribute__((ext_vector_type(4)));
typedef float fv2 __attribute__((ext_vector_type(2)));
template <int CPT>
struct FVec;
template <>
struct FVec<4> { using type = fv4; };
template <>
struct FVec<2> { using type = fv2; };
template <>
struct FVec<1> { using type = float; };

template <int CPT>
__device__ __forceinline__ void load_vec(const float* p, float (&v)[CPT]) {
  const typename FVec<CPT>::type t =
      __builtin_nontemporal_load(reinterpret_cast<const typename FVec<CPT>::type*>(p));
  __builtin_memcpy(v, &t, sizeof(t));
}

// The low bytes of a, b, c, d as one word, a lowest (byte selects: v_perm_b32
// takes bytes 0-3 from its second operand, 4-7 from its first, 0x0c = zero).
__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  const uint32_t lo = __builtin_amdgcn_perm((uint32_t)b, (uint32_t)a, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm((uint32_t)d, (uint32_t)c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// w with its byte c (0..3; a constant after unrolling) replaced by the low
// byte of v: select 4 + i (w's byte i) everywhere but byte c, which selects 0.
__device__ __forceinline__ uint32_t put_byte(uint32_t w, uint32_t v, int c) {
  return __builtin_amdgcn_perm(w, v, 0x07060504u & ~(0xFFu << (8 * c)));
}

// Stores the RT codes of one lane (RT = 8, 16 or 32 consecutive bytes).
template <int RT>
__device__ __forceinline__ void store_codes(int8_t* dst, const int (&q)[RT]) {
  if constexpr (RT == 8) {
    int2 o;
    o.x = (int)pack4(q[0], q[1], q[2], q[3]);
    o.y = (int)pack4(q[4], q[5], q[6], q[7]);
    *reinterpret_cast<int2*>(dst) = o;
  } else {
#pragma unroll
    for (int v = 0; v < RT / 16; ++v) {
      int4 o;
      o.x = (int)pack4(q[16 * v + 0], q[16 * v + 1], q[16 * v + 2], q[16 * v + 3]);
      o.y = (int)pack4(q[16 * v + 4], q[16 * v + 5], q[16 * v + 6], q[16 * v + 7]);
      o.z = (int)pack4(q[16 * v + 8], q[16 * v + 9], q[16 * v + 10], q[16 * v + 11]);
      o.w = (int)pack4(q[16 * v + 12], q[16 * v + 13], q[16 * v + 14], q[16 * v + 15]);
      reinterpret_cast<int4*>(dst)[v] = o;
    }
  }
}

// Stores RT bytes packed four to a word (RT = 8, 16 or 32).
template <int RT>
__device__ __forceinline__ void store_words(int8_t* dst, const uint32_t (&w)[RT / 4]) {
  if constexpr (RT == 8) {
    *reinterpret_cast<int2*>(dst) = make_int2((int)w[0], (int)w[1]);
  } else {
#pragma unroll
    for (int v = 0; v < RT / 16; ++v)
      reinterpret_cast<int4*>(dst)[v] = make_int4((int)w[4 * v], (int)w[4 * v + 1], (int)w[4 * v + 2], (int)w[4 * v + 3]);
  }
}

// PoT of a sub-channel maximum m ≥ 0 against a normal base in [2^-100, 2^100]:
// the smallest j in [0, 21] with m ≤ base·2^j (21 if none).  With
// m = 1.f_m·2^e_m and base = 1.f_b·2^e_b (base·2^j stays normal for j ≤ 21),
// m ≤ base·2^j holds exactly when j ≥ e_m − e_b + [f_m > f_b]; a zero or
// subnormal m gives j ≤ 0.  The same integer as counting the edges
// base·2^j (j = 0..20) below m.
__device__ __forceinline__ int pot_of(float m, float base) {
  const uint32_t bm = __float_as_uint(m), bb = __float_as_uint(base);
  const int j = (int)(bm >> 23) - (int)(bb >> 23) + ((bm & 0x7FFFFFu) > (bb & 0x7FFFFFu) ? 1 : 0);
  return min(max(j, 0), DSTAR_FMDQ_POT_MAX);
}

// A work item is kGroups consecutive (tile, channel group) pairs of the
// flattened [n_t][K / CPT] space, so no lane idles at the end of a tile's
// channels (with 512-channel slabs, K = 1152 left a quarter of the lanes idle).
template <int T, int CPT, int RT>
__global__ __launch_bounds__(kThreads, 2) void quantize_kernel(QuantizeArgs a, int64_t n_work,
                                                            int64_t n_groups) {
  constexpr int G = T / RT;                  // lanes per (tile, channels) group
  constexpr int kGroups = kThreads / G;      // channel groups per workgroup
  uint32_t hist[4] = {0u, 0u, 0u, 0u};
  const int64_t K = a.K;
  // The base: static (from the host), or the dynamic one in device memory,
  // whose reciprocal is formed here exactly as the host forms it.
  float base = a.base, inv_base = a.inv_base;
  if (a.base_dev != nullptr) {
    base = *a.base_dev;
    inv_base = (float)(1.0 / (double)base);
  }
  const int sub = threadIdx.x % G;           // which 16 rows of the tile
  const int grp = threadIdx.x / G;
  const int64_t kg_per_tile = K / CPT;       // CPT divides K
  for (int64_t wi = blockIdx.x; wi < n_work; wi += gridDim.x) {
    const int64_t g = wi * kGroups + grp;
    if (g >= n_groups) continue;             // the lanes of a group leave together
    const int64_t tile = g / kg_per_tile;
    const int64_t k = (g - tile * kg_per_tile) * CPT;
    const int64_t r0 = tile * T + sub * RT;  // first row of this lane
    const int64_t nrows = a.rows - r0;       // real rows from r0 (may be <= 0)

    // Δ = X_t − X_{t−1} for RT rows × CPT channels (Eq. 1), kept in registers.
    // The loads are unconditional, so all 2·RT of them are in flight together:
    // in a ragged last tile a row past the end reads the last row and is
    // zeroed after; every other tile takes the path without those selects.
    float d[RT][CPT];
    if (nrows >= RT) {
      const float* pt = a.x_t + r0 * K + k;
      const float* pp = a.x_prev + r0 * K + k;
      float xt[RT][CPT], xp[RT][CPT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        load_vec<CPT>(pt + t * K, xt[t]);
        load_vec<CPT>(pp + t * K, xp[t]);
      }
      // every load issued before the first use (otherwise the compiler waits
      // for each row's pair before issuing the next)
      __asm__ __volatile__("" ::: "memory");
#pragma unroll
      for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) d[t][c] = __fsub_rn(xt[t][c], xp[t][c]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int64_t r = min(r0 + t, a.rows - 1);
        float xt[CPT], xp[CPT];
        load_vec<CPT>(a.x_t + r * K + k, xt);
        load_vec<CPT>(a.x_prev + r * K + k, xp);
#pragma unroll
        for (int c = 0; c < CPT; ++c) d[t][c] = t < nrows ? __fsub_rn(xt[c], xp[c]) : 0.0f;
      }
    }

    uint32_t tagword = 0;
    // Aligned codes of the CPT channels, one packed word per row (q·2^e when
    // PoT ≤ 6, else its low digit): the 8-bit operand of stage 3's dense GEMM.
    uint32_t arow[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) arow[t] = 0u;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      // M: largest |Δ| of the sub-channel (QPU stage 1): this lane's rows,
      // then the other lanes' of the group.
      float m = 0.0f;
#pragma unroll
      for (int t = 0; t < RT; ++t) m = fmaxf(m, fabsf(d[t][c]));
#pragma unroll
      for (int o = 1; o < G; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      // PoT = number of bin edges base*2^j (j = 0..20) strictly below M, i.e.
      // the smallest j with M <= base*2^j, capped at 21 (Eq. 3; QPU stage 2),
      // read from the float fields instead of 21 compares.
      const int pot = pot_of(m, base);
      // Precision from the thresholds base*2^(k0+2N): p = b - 2 = log2(PCeil).
      const int p = pot <= a.k0 ? 0 : pot <= a.k0 + 2 ? 2 : pot <= a.k0 + 4 ? 4 : 6;
      const int e = pot - p;                               // step = base * 2^e
      const float scale = __int_as_float((127 - e) << 23);  // 2^-e, exact
      const float pceil = (float)(1 << p);
      int q[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        float r = __fmul_rn(__fmul_rn(d[t][c], inv_base), scale);
        r = __builtin_amdgcn_fmed3f(rintf(r), -pceil, pceil);   // clip to ±PCeil (r is finite)
        q[t] = (int)r;
      }
      // This lane's RT codes of channel k+c: bytes sub*RT .. sub*RT+RT-1 of
      // the channel's run at codes[(tile*K + k + c)*T].
      const int64_t run = (tile * K + k + c) * T + sub * RT;
      if (a.codes != nullptr) store_codes<RT>(a.codes + run, q);
      if (pot <= 6) {
#pragma unroll
        for (int t = 0; t < RT; ++t) arow[t] = put_byte(arow[t], (uint32_t)q[t] << e, c);
      } else if (a.acodes != nullptr) {
        // Digits of a = q·2^e (|a| ≤ 2^21): d0 in [−64, 63], d1 in
        // [−128, 127], d2 (0 unless PoT ≥ 14), packed as they are formed.
        uint32_t w1[RT / 4], w2[RT / 4];
#pragma unroll
        for (int v = 0; v < RT / 4; ++v) w1[v] = w2[v] = 0u;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int av = q[t] * (1 << e);
          const int d0 = ((av + 64) & 127) - 64;
          const int r1 = (av - d0) >> 7;
          const int d1 = ((r1 + 128) & 255) - 128;
          const int d2 = (r1 - d1) >> 8;
          arow[t] |= ((uint32_t)d0 & 0xFFu) << (8 * c);
          w1[t / 4] |= ((uint32_t)d1 & 0xFFu) << (8 * (t % 4));
          w2[t / 4] |= ((uint32_t)d2 & 0xFFu) << (8 * (t % 4));
        }
        store_words<RT>(a.hcodes + run, w1);
        if (pot > 13) store_words<RT>(a.hcodes + a.plane + run, w2);
      }
      if (sub == 0) hist[p >> 1] += 1u;
      const uint32_t tag = (uint32_t)(DSTAR_FMDQ_TAG_OFFSET - e) | ((uint32_t)(p >> 1) << DSTAR_FMDQ_PREC_SHIFT);
      tagword |= tag << (8 * c);
    }
    if (a.acodes != nullptr) {
      int8_t* ap = a.acodes + r0 * K + k;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        if constexpr (CPT == 4) {
          *reinterpret_cast<uint32_t*>(ap + t * K) = arow[t];
        } else if constexpr (CPT == 2) {
          *reinterpret_cast<uint16_t*>(ap + t * K) = (uint16_t)arow[t];
        } else {
          ap[t * K] = (int8_t)arow[t];
        }
      }
    }
    if (sub == 0) {
      uint8_t* tp = a.tags + tile * K + k;
      if constexpr (CPT == 4) {
        *reinterpret_cast<uint32_t*>(tp) = tagword;
      } else if constexpr (CPT == 2) {
        *reinterpret_cast<uint16_t*>(tp) = (uint16_t)tagword;
      } else {
        *tp = (uint8_t)tagword;
      }
    }
  }

  if (a.bit_hist == nullptr) return;
  // Block-wide histogram reduction, then at most four atomics per block.
  __shared__ uint32_t part[kThreads / 64][4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t v = hist[b];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6][b] = v;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    uint32_t v = 0;
    for (int w = 0; w < kThreads / 64; ++w) v += part[w][threadIdx.x];
    if (v) atomicAdd(a.bit_hist + threadIdx.x, v);
  }
}

template <int T, int CPT, int RT>
int launch_t(const QuantizeArgs& a, hipStream_t s) {
  constexpr int kGroups = kThreads / (T / RT);
  const int64_t nt = n_tiles(a.rows, T);
  const int64_t n_groups = nt * (a.K / CPT);
  const int64_t n_work = (n_groups + kGroups - 1) / kGroups;
  const int64_t grid = n_work < kMaxGrid ? n_work : kMaxGrid;
  hipLaunchKernelGGL((quantize_kernel<T, CPT, RT>), dim3((unsigned)grid), dim3(kThreads), 0, s, a,
                     n_work, n_groups);
  return check_launch("fmdq_quantize");
}

}  // namespace

int launch_quantize(const QuantizeArgs& a, hipStream_t s) {
  if (a.rows == 0) return DSTAR_OK;
  // Channels per lane group: up to 4 as K's divisibility allows (16 · CPT
  // floats of Δ live in each lane's registers; two waves per SIMD).  At T = 32
  // two channels per group (smaller slabs, more workgroups) measured slower in
  // the pipelined step.
  const bool vec4 = (a.K % 4) == 0;
  const bool vec2 = (a.K % 2) == 0;
  switch (a.T) {
    case 16:
      return vec4 ? launch_t<16, 4, RT>(a, s) : vec2 ? launch_t<16, 2, RT>(a, s) : launch_t<16, 1, RT>(a, s);
    case 32:
      // Below 256 workgroups the launch is one short pass whose length is a
      // lane's chain of row loads: 8 rows per lane (four lanes per group,
      // twice the workgroups) shortens it (DiT-XL/2 layer 7.6 -> 7.2 us).
      if (vec4 && (n_tiles(a.rows, 32) * (a.K / 4) + 127) / 128 < 256) return launch_t<32, 4, 8>(a, s);
      return vec4 ? launch_t<32, 4, RT>(a, s) : vec2 ? launch_t<32, 2, RT>(a, s) : launch_t<32, 1, RT>(a, s);
    case 64:
      return vec4 ? launch_t<64, 4, RT>(a, s) : vec2 ? launch_t<64, 2, RT>(a, s) : launch_t<64, 1, RT>(a, s);
    default:
      return set_error(DSTAR_EUNSUPPORTED, "token_tile %d not supported", a.T);
  }
}

}  // namespace dstar
