/*
 * Sparse Attention Reuse (SAR) with FMDQ-INT8 operands: C ABI.
 *
 * Source: "DSTAR: Accelerating Diffusion Transformers via Spatial and Temporal
 * Redundancy Reduction" (arXiv 2607.15846), §3.2 "Sparse Attention Reuse"
 * (Fig. 8: cached and reused steps), §4.3 "Attention Operation" (Fig. 13:
 * block-sparse schedule, INT8 products, FMDQ on the activations).
 *
 * One attention layer of B images × H heads over L tokens with head width d.
 * A static block mask per head (64 × 64 blocks, found offline) keeps some
 * (query block, key block) pairs.  The cached step quantizes Q, K and V,
 * computes the kept blocks of the scores, their row softmax and the FMDQ-INT8
 * codes of the attention weights P (the cache), then O = P V.  A reused step
 * quantizes the current V and computes O = P_cache V.
 *
 * Operands (see each entry point for the exact rounding):
 *   Q: FMDQ at 8 bits: one PoT per (32-row token tile, channel) sub-channel
 *      against the static base_q, codes in [-64, 64] (§3.1 Eq. 2-5);
 *   K: int8 with one scale per key,     scale = fl32(max|K[s][:]| / 127);
 *   V: int8 with one scale per channel, scale = fl32(max|V[:][c]| / 127);
 *   P: FMDQ at 8 bits per (32-row tile, key) sub-channel against base_p.
 * Every product is an exact integer sum; logits, softmax and outputs are
 * formed from it in a fixed sequence of float32/float64 roundings.
 *
 * Layouts (all device memory, owned by the caller; BH = B·H, rows of one
 * (image, head) pair are contiguous, batch-major then head):
 *   q, k, v      float32 [BH][L][d]
 *   qcodes       int8    [BH][L][dp]      dp = d rounded up to a multiple of 32;
 *   kcodes       int8    [BH][L][dp]      channels d..dp-1 are written 0
 *   qpot         uint8   [BH][L/32][dp]   PoT of each Q sub-channel (0..21)
 *   kscale       float32 [BH][L]
 *   vcodes_t     int8    [BH][dp][L]      V codes transposed (channel-major)
 *   vscale       float32 [BH][d]
 *   row_ptr      int32   [H·(L/64) + 1]   compressed rows of the block mask,
 *   cols         int32   [nnz]            row = (head, query block), columns =
 *                                          kept key blocks (ascending)
 *   pcodes       int8    [B][nnz][64][64] cache: P codes of kept block j
 *                                          ([query row in block][key in block])
 *   ppot         uint8   [B][nnz][2][64]  cache: PoT per (token tile, key)
 *   out          float32 [BH][L][d]
 * Column entries outside [0, L/64) and row_ptr entries outside [0, nnz] are
 * ignored (clamped); a query block without kept key blocks gets O = 0.
 *
 * Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 * stream), allocates nothing and keeps no state.  Return values and
 * dstar_fmdq_last_error() as in dstar_fmdq.h.  Alignment: int8/uint8 arrays
 * 16 bytes, float arrays 4 bytes (DSTAR_EALIGN otherwise).
 */
#ifndef DSTAR_SAR_H
#define DSTAR_SAR_H

#include <stdint.h>

#include "dstar_fmdq.h"

#ifdef __cplusplus
extern "C" {
#endif

#define DSTAR_SAR_BLOCK 64     /* mask block edge, queries and keys */
#define DSTAR_SAR_TILE 32      /* FMDQ token tile of Q and P */
#define DSTAR_SAR_PAD 32       /* dp = round_up(d, DSTAR_SAR_PAD) */
#define DSTAR_SAR_MAX_D 128    /* head width limit */
#define DSTAR_SAR_MAX_L 65536  /* tokens per image limit */
#define DSTAR_SAR_EXP_FRAC 36  /* fixed-point fraction bits of the softmax numerators */

typedef struct {
  int32_t batch;     /* B >= 1 */
  int32_t heads;     /* H >= 1 */
  int32_t tokens;    /* L: a multiple of 64 in [64, DSTAR_SAR_MAX_L] */
  int32_t head_dim;  /* d in [1, DSTAR_SAR_MAX_D] */
  float base_q;      /* static FMDQ base of Q, in [2^-100, 2^100] */
  float base_p;      /* static FMDQ base of P, in [2^-100, 2^100] */
  float sm_scale;    /* logit scale (usually 1/sqrt(d)), finite and > 0 */
} dstar_sar_params;

/* FMDQ-INT8 of Q (§3.1 Eq. 2-5 at 8 bits; §4.3 "quantization on
 * activations using FMDQ, with INT8 precision").  Per sub-channel (32-row
 * tile τ, channel c): M = max |Q|; PoT = the smallest j in [0, 21] with
 * M <= fl32(base_q·2^j) (21 if none); e = PoT − 6; code =
 * clip(rint(fl32(fl32(Q·inv)·2^-e)), -64, 64) with inv = fl32(1/f64(base_q)).
 * Writes qcodes and qpot. */
int dstar_sar_quantize_q(const dstar_sar_params* p, const float* q, int8_t* qcodes, uint8_t* qpot,
                         void* stream);

/* int8 of K with one scale per key (the output columns of Q·K^T; the 8-bit
 * weight operand of the MPU, §4.2): scale = fl32(f64(max_c |K[s][c]|) / 127),
 * code = clip(rint(f64(K) / f64(scale)), -127, 127), 0 where scale = 0. */
int dstar_sar_quantize_k(const dstar_sar_params* p, const float* k, int8_t* kcodes, float* kscale,
                         void* stream);

/* int8 of V with one scale per head channel (the output columns of P·V), as
 * for K with the maximum taken over the L keys; codes written transposed.
 * vscale is also the reduction's workspace (overwritten). */
int dstar_sar_quantize_v(const dstar_sar_params* p, const float* v, int8_t* vcodes_t, float* vscale,
                         void* stream);

/* Cached step, scores to cache (§3.2 Fig. 8 cached step; §4.3 Fig. 13(a)).
 * For each kept block, with a_Q = code·2^PoT:
 *   S_int[t][s] = Σ_c a_Q[t][c]·kcode[s][c]                     (exact)
 *   z = fl32(f64(S_int)·f_s),  f_s = f64(kscale[s])·((f64(base_q)·2^-6)·f64(sm_scale))
 * Row softmax over all kept keys of the query row:
 *   x = fl32(z − max z); e = exp32(x) (Cody–Waite reduction, degree-7 Taylor
 *   polynomial, float32, fixed rounding order; 0 for x < -26);
 *   E = rint(e·2^36) (integer); P = fl32(f64(E)·(1/f64(Σ E))).
 * FMDQ-INT8 of P per (32-row tile, key) sub-channel against base_p as for Q.
 * Writes pcodes and ppot of every kept block. */
int dstar_sar_scores(const dstar_sar_params* p, const int32_t* row_ptr, const int32_t* cols, int32_t nnz,
                     const int8_t* qcodes, const uint8_t* qpot, const int8_t* kcodes, const float* kscale,
                     int8_t* pcodes, uint8_t* ppot, void* stream);

/* O = P·V over the kept blocks (§3.2 cached and reused steps; §4.3 Fig.
 * 13(b)), with a_P = pcode·2^PoT:
 *   O_int[t][c] = Σ_{kept s} a_P[t][s]·vcode[s][c]                (exact)
 *   O = fl32(f64(O_int)·(f64(vscale[c])·(f64(base_p)·2^-6)))
 * Writes every element of out. */
int dstar_sar_pv(const dstar_sar_params* p, const int32_t* row_ptr, const int32_t* cols, int32_t nnz,
                 const int8_t* pcodes, const uint8_t* ppot, const int8_t* vcodes_t, const float* vscale,
                 float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSTAR_SAR_H */
