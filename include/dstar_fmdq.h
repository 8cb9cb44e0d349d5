/*
 * dstar_fmdq.h — C ABI of the FMDQ differential linear layer on AMD Instinct
 * MI355X (gfx950).
 *
 * Method: "DSTAR: Accelerating Diffusion Transformers via Spatial and Temporal
 * Redundancy Reduction" (arXiv 2607.15846), cited as DSTAR.  For two adjacent
 * denoising timesteps a linear layer y = W x is updated differentially
 * (DSTAR §2.2, Eq. 1): Y_t = Y_{t-1} + W·(X_t − X_{t-1}).  The difference Δ is
 * quantized per sub-channel (token tile × input channel) with power-of-two
 * scales relative to a static base (DSTAR §3.1 step 1, Eq. 2–5), the channels
 * of each token tile are grouped by their fused precision/scale tag (FPoT,
 * DSTAR §3.1 step 3), each group is multiplied by int8 weights into its own
 * integer accumulator, the group sums are aligned by left shifts (DSTAR §3.1
 * steps 2 and 5, Fig. 6), dequantized and added to the cached Y_{t-1} (DSTAR
 * §4.2 "Design of MPU", §4.3 "Linear Operation").
 *
 * The entry points are the three stages, the weight preparation, the
 * one-call layer (with a workspace, or without one) and the variants (dynamic
 * base, fused GELU, 2-bit slice stream); each launches HIP kernels on the
 * caller's stream and returns without synchronizing.
 *
 * Compared with a minimal three-call interface (stage 1 writing codes and
 * tags; stage 2 writing channel ids sorted by (tag, channel) with 17 tag
 * offsets; stage 3 taking codes, tags, ids, offsets and W):
 *   - stage 1 also writes the shift-aligned codes and their high digits
 *     (acodes, hcodes), the operands of the MFMA kernels (DSTAR §3.1 step 5:
 *     the alignment is applied to the codes before the multiply), and may
 *     then leave out the plain codes, which only the per-group kernel reads;
 *   - stage 2 orders ties inside one tag by precision, widest first, then by
 *     channel, and writes 65 offsets, one per (tag, precision) bin plus the
 *     end (DSTAR §3.1 step 3 fixes only the tag order);
 *   - stage 3 takes no tags (a channel's group and precision follow from its
 *     position in perm against the bin offsets), takes acodes, hcodes and a
 *     once-per-layer W^T (dstar_fmdq_pack_weights), accepts any int8 weight,
 *     -128 included, and can dump its exact integer S (s_dbg);
 *   - the stream is a hipStream_t passed as void*, so this header needs no
 *     HIP header.
 *
 * Conventions for every entry point
 *   - All array arguments are DEVICE pointers (memory from hipMalloc, or
 *     torch CUDA tensors on ROCm), owned by the caller.  The library keeps no
 *     reference to them after the call returns and allocates no memory.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *   - Return value: DSTAR_OK (0), or a negative DSTAR_E* code.  On error no
 *     kernel was launched (except DSTAR_EHIP, reported after a failed launch)
 *     and dstar_fmdq_last_error() describes the cause (thread-local string).
 *   - Argument checks happen on the host before any HIP call, so invalid
 *     arguments are reported even on a machine without a GPU.
 *   - Inputs must be finite; results for NaN/Inf inputs are unspecified.
 *   - Only y_out may alias y_prev; no other arguments may overlap.
 */
#ifndef DSTAR_FMDQ_H
#define DSTAR_FMDQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSTAR_FMDQ_ABI_VERSION 10  /* also covers the entry points of dstar_sar.h */

/* Rule constants (DSTAR §3.1 step 1; readings in the design notes):
 * PCeil of a b-bit sub-channel is 2^(b-2); PoT is capped at POT_MAX so that
 * the tag (b-2) - PoT + TAG_OFFSET always lies in [0, NUM_TAGS). */
#define DSTAR_FMDQ_NUM_TAGS 16
#define DSTAR_FMDQ_NUM_BINS 64 /* (tag, precision) bins of the bucket order */
#define DSTAR_FMDQ_TAG_OFFSET 15
#define DSTAR_FMDQ_POT_MAX 21
#define DSTAR_FMDQ_PREC_SHIFT 4
#define DSTAR_FMDQ_MAX_K 65535
#define DSTAR_FMDQ_SLICE_BINS 22     /* slice tags -6..15 of the 2-bit stream */
#define DSTAR_FMDQ_SLICE_TAG_OFFSET 6
#define DSTAR_FMDQ_SLICE_MAX_K 16384
#define DSTAR_FMDQ_NOALLOC_MAX_BYTES (64 << 20) /* scratch of dstar_fmdq_layer_noalloc */

/* Status codes. */
#define DSTAR_OK 0
#define DSTAR_EINVAL (-1)       /* a size or parameter is out of range       */
#define DSTAR_ENULL (-2)        /* a required pointer is NULL                */
#define DSTAR_EALIGN (-3)       /* a pointer is not aligned as required      */
#define DSTAR_EUNSUPPORTED (-4) /* valid for the method, not supported here  */
#define DSTAR_EHIP (-5)         /* the HIP runtime reported an error         */

/* Layer parameters shared by the three stages.
 *   rows            M = batch * tokens, rows of X and Y (batch-major), >= 0.
 *   tokens_per_seq  tokens of one sequence; token tiles never straddle two
 *                   sequences, so rows must equal tokens_per_seq (one
 *                   sequence, last tile may be ragged) or be a multiple of it
 *                   with tokens_per_seq % token_tile == 0.
 *   K               input channels, 1..65535 (channel ids are uint16).
 *   token_tile      T, rows per token tile: 16, 32 or 64 (DSTAR §3.1 step 1
 *                   tiles Δ along the token dimension).
 *   base            static per-layer base scale (DSTAR §3.1: fixed ahead of
 *                   time instead of taken from the data), a normal float in [2^-100, 2^100].
 *   thr0_log2       k0 in Thr_0 = base * 2^k0, the 2-bit threshold of the
 *                   precision bins Thr_0 * 4^N (DSTAR §3.1 step 1), 1..15.
 * Tiles: n_t = ceil(rows / T); tile τ holds rows [τT, min(τT+T, rows)). */
typedef struct {
  int32_t rows;
  int32_t tokens_per_seq;
  int32_t K;
  int32_t token_tile;
  float base;
  int32_t thr0_log2;
} dstar_fmdq_params;

/* Stage 1 — differential + sub-channel quantization (DSTAR Eq. 1; §3.1 step
 * 1, Eq. 2-5; §4.2 QPU stages 1-3).
 *   x_t, x_prev  [rows][K] float32 row-major, 16-byte aligned.
 *   codes        [n_t][K][T] int8 (out): code of row τT+t, channel k at
 *                codes[(τK + k)T + t]; rows past the end of a ragged last tile
 *                are written 0.  16-byte aligned.  May be NULL when acodes
 *                and hcodes are given (they hold the same codes, aligned);
 *                NULL without them is DSTAR_ENULL.
 *   tags         [n_t][K] uint8 (out), 4-byte aligned: bits 0-3 the FPoT tag
 *                g = (b-2) - PoT + 15 (ascending g = ascending FPoT; the
 *                sub-channel's step is base * 2^(15-g)), bits 4-5 the
 *                precision code b/2 - 1.
 *   acodes       NULL, or [n_t*T][K] int8 row-major (out), 16-byte aligned:
 *                the shift-aligned operand of stage 3's dense GEMM (DSTAR
 *                §3.1 step 5: partial sums of different FPoT are aligned by
 *                left shifts; here the codes are shifted before the multiply).
 *                With a = code * 2^(15-g), the code in units of the base
 *                (|a| <= 2^PoT), split into signed digits
 *                a = d0 + 2^7*d1 + 2^15*d2 (d0 in [-64, 63], d1 in
 *                [-128, 127], d2 in [-64, 64]): acodes[τT+t][k] = a if
 *                PoT <= 6, else d0.  Rows past a ragged end are 0.
 *   hcodes       NULL (exactly when acodes is NULL), or [2][n_t][K][T] int8
 *                (out), 16-byte aligned, laid out like codes: plane 0 holds d1
 *                of every sub-channel with PoT >= 7, plane 1 holds d2 of
 *                every sub-channel with PoT >= 14.  All other entries are
 *                left unwritten.
 *   bit_hist     uint32[4] or NULL: counts of sub-channels quantized at
 *                2/4/6/8 bits are ADDED to it (the caller zeroes it).
 * Per sub-channel: M = max |Δ| over the tile's rows; PoT = smallest j in
 * [0, 21] with M <= base*2^j (21 if none); bits = 2/4/6/8 for PoT <= k0,
 * k0+2, k0+4, else; e = PoT - (b-2); code = clip(rint(fl32(fl32(Δ *
 * fl32(1/base)) * 2^-e)), ±2^(b-2)). */
int dstar_fmdq_quantize(const dstar_fmdq_params* p, const float* x_t,
                        const float* x_prev, int8_t* codes, uint8_t* tags,
                        int8_t* acodes, int8_t* hcodes, uint32_t* bit_hist,
                        void* stream);

/* Stage 2 — reorder the channels of every token tile by FPoT (DSTAR §3.1
 * step 3; §4.2 QPU stage 4), as a stable counting sort over the 64 bins
 * bin = 4 * tag + (3 - precision code): FPoT tag ascending, inside one tag the
 * precision descending, then the channel ascending.  (The pages fix only the
 * FPoT order.  With the wider codes first, the sub-channels of a group whose
 * shift-aligned codes exceed 8 bits form a prefix of that group.)
 *   tags       [n_t][K] uint8 from stage 1.
 *   perm       [n_t][K] uint16 (out): channel ids of tile τ in that order.
 *   group_off  [n_t][65] int32 (out): group_off[τ][β] = number of channels of
 *              tile τ with bin < β (group_off[τ][64] = K).  FPoT group g is
 *              perm[τ][group_off[τ][4g] .. group_off[τ][4g+4]). */
int dstar_fmdq_bucket(const dstar_fmdq_params* p, const uint8_t* tags,
                      uint16_t* perm, int32_t* group_off, void* stream);

/* The 2-bit slice stream of DSTAR's accelerator (§3.1 steps 2-4: sub-channel
 * decomposition into 2-bit slices, reordering by FPoT, encoding of channel
 * indices and shift counts; §4.2 QPU stages 3-4).  For inspection and for a
 * 2-bit datapath: dstar_fmdq_linear does not read it.  K <= 16384.
 *   codes, tags  from stage 1.
 *   entries    [n_t][4K] uint32 (out), 4-byte aligned: the entries of tile τ,
 *              channel k | slice n << 16 | shift << 24, ordered by bin =
 *              tag - 2n + 6 (the slice's FPoT lowered by 2n) ascending, then
 *              channel ascending; shift = bin - previous entry's bin (0 for
 *              the first) = the left shift applied to the running partial sum
 *              before adding this entry's product.  A b-bit sub-channel gives
 *              b/2 entries (n = 0 .. b/2-1); entries past the tile's count are
 *              0xFFFFFFFF.
 *   slices     [n_t][4K][T/4] uint8 (out): entry j's 2-bit fields for rows t,
 *              four rows per byte (row t at bits 2*(t mod 4)); field = (code >>
 *              2n) & 3, i.e. the radix-4 digits of the two's-complement code,
 *              the top one (n = b/2-1) read as signed (-2..1), the others
 *              unsigned.  code = sum_n digit_n * 4^n.
 *   slice_off  [n_t][23] int32 (out): entries of tile τ with bin < β.
 * Decoding: acc <<= shift; acc += digits * W[k]; after the last entry
 * S = acc * 2^(15 - (bin_last - 6)). */
int dstar_fmdq_slice_encode(const dstar_fmdq_params* p, const int8_t* codes,
                            const uint8_t* tags, uint32_t* entries,
                            uint8_t* slices, int32_t* slice_off, void* stream);

/* Weight preparation, once per layer: w_t[n][k] = w[k][n] (the [out][in]
 * layout of the weights), the operand of stage 3's dense GEMM.
 *   w    [K][N] int8 row-major; w_t [N][K] int8 (out).  No alignment
 *        requirement beyond 16 bytes for both. */
int dstar_fmdq_pack_weights(int32_t K, int32_t N, const int8_t* w, int8_t* w_t,
                            void* stream);

/* Stage 3 — grouped int8 GEMM, shift alignment, dequantization and reverse
 * differential (DSTAR §3.1 steps 3 and 5, Fig. 6; §4.2 MPU, inverse
 * quantization and accumulation units; §4.3 reverse differential fused into
 * the GEMM).
 *   N          output channels, a multiple of 4 in [4, 2^20].
 *   codes      from stage 1; perm, group_off ([n_t][65]) from stage 2.
 *              Channel k of FPoT group g of tile τ is multiplied at step
 *              2^(15-g) * base.  codes may be NULL when acodes and hcodes
 *              are given and the MFMA kernel runs (below); a call that needs
 *              the per-group kernel (acc_dbg, no w_t, or a shape the MFMA
 *              kernels do not take) without codes returns DSTAR_ENULL.
 *   acodes     NULL, or stage 1's aligned codes.
 *   hcodes     NULL, or stage 1's digit planes (given with acodes).
 *   w          [K][N] int8 row-major, 16-byte aligned; any int8 value
 *              (-128 included).
 *   w_t        NULL, or the [N][K] copy made by dstar_fmdq_pack_weights.
 *   w_scale    [N] float32, per-output-channel weight scale.
 *   y_prev     [rows][N] float32, the cached output Y_{t-1}.
 *   y_out      [rows][N] float32 (out), Y_t; may equal y_prev (in place).
 *              y_prev and y_out are 16-byte aligned.
 *   acc_dbg    NULL, or [dbg_tile_hi - dbg_tile_lo][16][T][N] int32 (out): the
 *              group accumulators acc_g[t][n] = Σ over channels k of group g
 *              of code(τT+t, k) * w[k][n] for tiles τ in [dbg_tile_lo,
 *              dbg_tile_hi); groups absent from a tile and rows past a ragged
 *              end are written 0.  Needs 0 <= lo < hi <= n_t.  With acc_dbg
 *              the layer runs in the per-group kernel (slow; for checking):
 *              only that kernel keeps one accumulator per FPoT group.
 *   s_dbg      NULL, or [dbg_tile_hi - dbg_tile_lo][T][N] int64 (out),
 *              8-byte aligned: the exact integer S of every output of the
 *              tiles in [dbg_tile_lo, dbg_tile_hi) (0 on rows past a ragged
 *              end), as the kernel that computes the layer holds it before
 *              the dequantization: the MFMA kernel when acc_dbg is NULL and
 *              the shape allows it, else the per-group kernel.  For checking.
 * Per output: S = Σ_g acc_g * 2^(15-g) (an exact integer);
 * y_out = fl32(f64(y_prev) + (f64(S) * f64(base)) * f64(w_scale[n])).
 * With acodes, hcodes and w_t given (T of 16, 32 or 64, K % 16 == 0, K*N
 * below 2^31, n_t*K*T at most 2^30, N below 2^23) the MFMA kernel runs: S = acodes x w_t + 2^7 * (d1
 * digits x w) + 2^15 * (d2 digits x w), the digit terms over the channels
 * with PoT >= 7 (resp. >= 14) of each token tile, which are prefixes of the
 * FPoT groups in perm; a token tile whose int32 accumulator it cannot prove
 * exact (128 * Σ_k 2^PoT_k >= 2^31; |W| <= 128) is finished by an exact int64
 * path that rebuilds each channel's aligned value d0 + 2^7*d1 + 2^15*d2 from
 * acodes and hcodes, walking perm bin by bin (the bin fixes the PoT and so
 * which digits exist).  Otherwise the per-group kernel runs. */
int dstar_fmdq_linear(const dstar_fmdq_params* p, int32_t N,
                      const int8_t* codes, const uint16_t* perm,
                      const int32_t* group_off, const int8_t* acodes,
                      const int8_t* hcodes, const int8_t* w, const int8_t* w_t,
                      const float* w_scale,
                      const float* y_prev, float* y_out, int32_t* acc_dbg,
                      int64_t* s_dbg, int32_t dbg_tile_lo, int32_t dbg_tile_hi,
                      void* stream);

/* Stage 3 with the MLP activation fused into its epilogue (DSTAR §4.3
 * "Linear Operation": the GELU that follows the first linear of a DiT MLP is
 * applied by the vector unit as the output is produced; §4.2 "Design of
 * VPU").  Arguments and results as for dstar_fmdq_linear (without the
 * accumulator dump), plus
 *   gelu_out  [rows][N] float32 (out), 16-byte aligned, sharing no byte with
 *             y_prev or y_out (DSTAR_EINVAL otherwise): GELU(Y_t) for every output written to y_out, in the tanh
 *             form y / (1 + exp(-2u)), u = 0.7978845608028654 * (y + 0.044715 *
 *             (y*y)*y), evaluated in float64 and rounded once to float32 (the
 *             pages give no formula; their unit uses piecewise cubics).
 * In a chain of timesteps gelu_out is the second linear's X_t, and the
 * previous step's gelu_out its X_{t-1}. */
int dstar_fmdq_linear_gelu(const dstar_fmdq_params* p, int32_t N,
                           const int8_t* codes, const uint16_t* perm,
                           const int32_t* group_off, const int8_t* acodes,
                           const int8_t* hcodes, const int8_t* w,
                           const int8_t* w_t, const float* w_scale,
                           const float* y_prev, float* y_out, float* gelu_out,
                           void* stream);

/* Elementwise GELU, the same function as dstar_fmdq_linear_gelu's:
 * g[i] = GELU(y[i]) for i < n (n >= 0).  y and g are 16-byte aligned device
 * arrays; g may equal y.  For the GELU of a cached output, e.g. the second
 * linear's X_{t-1} when a chain of timesteps starts. */
int dstar_fmdq_gelu(const float* y, float* g, int64_t n, void* stream);

/* Dynamic base, pass 1 of the variant that takes the base from the data
 * (DSTAR §3.1 step 1 defines the base of Eq. 2-3 as the smallest sub-channel
 * maximum M_i over the whole tensor, which costs a second pass over X; the
 * method's static base removes it, and DSTAR §5.2, Table 2 evaluates the
 * dynamic variant as DS-FMDQ-DYN).
 *   x_t, x_prev  as for stage 1 (may be NULL when rows == 0).
 *   base         float32[1], DEVICE memory, 4-byte aligned (out): the smallest
 *                M = max |Δ| over the rows of a token tile, over every
 *                sub-channel with M > 0, clamped to [2^-100, 2^100]; p->base
 *                when no sub-channel has M > 0.
 * The result stays on the device for the _dyn entry points below (three
 * kernels; no memset, so the sequence can be captured in a HIP graph). */
int dstar_fmdq_dynamic_base(const dstar_fmdq_params* p, const float* x_t,
                            const float* x_prev, float* base, void* stream);

/* Stage 1 and stage 3 with the base read from device memory: `base` is a
 * float32[1] written by dstar_fmdq_dynamic_base (or any float in
 * [2^-100, 2^100]), 4-byte aligned, not NULL.  Every other argument, check
 * and result is that of dstar_fmdq_quantize, resp. dstar_fmdq_linear, with
 * p->base replaced by *base (p->base must still be valid).  Stage 2 does not
 * depend on the base. */
int dstar_fmdq_quantize_dyn(const dstar_fmdq_params* p, const float* base,
                            const float* x_t, const float* x_prev,
                            int8_t* codes, uint8_t* tags, int8_t* acodes,
                            int8_t* hcodes, uint32_t* bit_hist, void* stream);
int dstar_fmdq_linear_dyn(const dstar_fmdq_params* p, const float* base,
                          int32_t N, const int8_t* codes, const uint16_t* perm,
                          const int32_t* group_off, const int8_t* acodes,
                          const int8_t* hcodes, const int8_t* w,
                          const int8_t* w_t, const float* w_scale,
                          const float* y_prev, float* y_out, int32_t* acc_dbg,
                          int64_t* s_dbg, int32_t dbg_tile_lo,
                          int32_t dbg_tile_hi, void* stream);

/* The whole layer in one call: stages 1, 2 and 3 (dstar_fmdq_quantize with
 * the aligned codes and digit planes, dstar_fmdq_bucket, dstar_fmdq_linear)
 * on `stream`, with every intermediate (codes, tags, aligned codes, digit
 * planes, bucket ids and bin offsets) in a caller workspace (DSTAR §3.1 steps
 * 1-5; §4.3 "Linear Operation": quantization, reorder and the GEMM with its
 * fused reverse differential as one pipelined operation).
 *   x_t, x_prev, w, w_t, w_scale, y_prev, y_out, bit_hist  as for the stages
 *              (w_t may be NULL: then the per-group kernel runs).
 *   workspace  device memory, 256-byte aligned, of at least
 *              dstar_fmdq_layer_workspace_size(p) bytes; its contents on entry
 *              do not matter, and it holds the intermediates afterwards.
 *              Two calls that share a workspace must not overlap in time.
 * Errors as for the stages, plus DSTAR_EINVAL when workspace_bytes is too
 * small.  The library allocates nothing. */
int dstar_fmdq_layer(const dstar_fmdq_params* p, int32_t N, const float* x_t,
                     const float* x_prev, const int8_t* w, const int8_t* w_t,
                     const float* w_scale, const float* y_prev, float* y_out,
                     uint32_t* bit_hist, void* workspace, int64_t workspace_bytes,
                     void* stream);

/* Bytes of workspace dstar_fmdq_layer needs for these parameters (>= 0), or a
 * negative DSTAR_E* code for invalid parameters. */
int64_t dstar_fmdq_layer_workspace_size(const dstar_fmdq_params* p);

/* dstar_fmdq_layer without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The intermediates live in the library's
 * own device array of DSTAR_FMDQ_NOALLOC_MAX_BYTES (64 MiB), one per GPU, held
 * until the process ends; its address on a device is looked up once, on the
 * first call there.  Arguments, results and errors as for dstar_fmdq_layer,
 * plus DSTAR_EINVAL (before any HIP call) when
 * dstar_fmdq_layer_workspace_size(p) exceeds that size.  Nothing is
 * allocated.  Every call on one GPU uses the same array: calls that overlap in
 * time on one GPU (on different streams, or from different threads) race and
 * must be serialized by the caller.  Nothing needs clearing between calls:
 * the stages write every intermediate they read. */
int dstar_fmdq_layer_noalloc(const dstar_fmdq_params* p, int32_t N,
                             const float* x_t, const float* x_prev,
                             const int8_t* w, const int8_t* w_t,
                             const float* w_scale, const float* y_prev,
                             float* y_out, uint32_t* bit_hist, void* stream);

/* Message describing the last error of the calling thread ("" if none). */
const char* dstar_fmdq_last_error(void);

/* DSTAR_FMDQ_ABI_VERSION of the library. */
int dstar_fmdq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSTAR_FMDQ_H */
