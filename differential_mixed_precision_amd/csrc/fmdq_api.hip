// C ABI of the FMDQ differential linear (declared in include/dstar_fmdq.h):
// host-side argument checks, then the stream-ordered kernel launches.
#include <cmath>
#include <cstring>
#include <string>

#include "fmdq_internal.h"

namespace dstar {

namespace {
thread_local std::string g_error;

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Checks the parameters shared by all stages; fills n_t.
int check_params(const dstar_fmdq_params* p, int64_t* nt) {
  if (p == nullptr) return set_error(DSTAR_ENULL, "params is NULL");
  if (p->rows < 0) return set_error(DSTAR_EINVAL, "rows = %d < 0", p->rows);
  if (p->K < 1 || p->K > DSTAR_FMDQ_MAX_K)
    return set_error(DSTAR_EINVAL, "K = %d outside [1, %d]", p->K, DSTAR_FMDQ_MAX_K);
  if (p->token_tile != 16 && p->token_tile != 32 && p->token_tile != 64)
    return set_error(DSTAR_EINVAL, "token_tile = %d not in {16, 32, 64}", p->token_tile);
  if (p->tokens_per_seq < 1)
    return set_error(DSTAR_EINVAL, "tokens_per_seq = %d < 1", p->tokens_per_seq);
  if (p->rows > p->tokens_per_seq &&
      (p->rows % p->tokens_per_seq != 0 || p->tokens_per_seq % p->token_tile != 0))
    return set_error(DSTAR_EINVAL,
                     "rows = %d spans several sequences of %d tokens: rows must be a multiple of "
                     "tokens_per_seq and tokens_per_seq a multiple of token_tile = %d",
                     p->rows, p->tokens_per_seq, p->token_tile);
  const float b = p->base;
  if (!std::isfinite(b) || !(b >= std::ldexp(1.0f, -100)) || !(b <= std::ldexp(1.0f, 100)))
    return set_error(DSTAR_EINVAL, "base = %g outside [2^-100, 2^100]", (double)b);
  if (p->thr0_log2 < 1 || p->thr0_log2 > 15)
    return set_error(DSTAR_EINVAL, "thr0_log2 = %d outside [1, 15]", p->thr0_log2);
  *nt = n_tiles(p->rows, p->token_tile);
  return DSTAR_OK;
}
}  // namespace

int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

void clear_error() { g_error.clear(); }

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DSTAR_EHIP, "%s: %s", what, hipGetErrorString(e));
  return DSTAR_OK;
}

}  // namespace dstar

using namespace dstar;

extern "C" {

int dstar_fmdq_abi_version(void) { return DSTAR_FMDQ_ABI_VERSION; }

const char* dstar_fmdq_last_error(void) { return g_error.c_str(); }

}  // extern "C"

namespace {

int quantize_impl(const dstar_fmdq_params* p, const float* base_dev, const float* x_t,
                  const float* x_prev, int8_t* codes, uint8_t* tags, int8_t* acodes,
                  int8_t* hcodes, uint32_t* bit_hist, void* stream) {
  clear_error();
  int64_t nt = 0;
  if (int rc = check_params(p, &nt)) return rc;
  if (p->rows == 0) return DSTAR_OK;
  if (!x_t || !x_prev || !tags)
    return set_error(DSTAR_ENULL, "quantize: x_t, x_prev and tags must not be NULL");
  if (!codes && !acodes)
    return set_error(DSTAR_ENULL, "quantize: codes may be NULL only when acodes and hcodes are given");
  if (!aligned(x_t, 16) || !aligned(x_prev, 16) || (codes && !aligned(codes, 16)) || !aligned(tags, 4))
    return set_error(DSTAR_EALIGN,
                     "quantize: x_t, x_prev and codes must be 16-byte aligned, tags 4-byte aligned");
  if (bit_hist && !aligned(bit_hist, 4))
    return set_error(DSTAR_EALIGN, "quantize: bit_hist must be 4-byte aligned");
  if ((acodes == nullptr) != (hcodes == nullptr))
    return set_error(DSTAR_ENULL, "quantize: acodes and hcodes must both be given or both be NULL");
  if ((acodes && !aligned(acodes, 16)) || (hcodes && !aligned(hcodes, 16)))
    return set_error(DSTAR_EALIGN, "quantize: acodes and hcodes must be 16-byte aligned");
  QuantizeArgs a;
  a.x_t = x_t;
  a.x_prev = x_prev;
  a.codes = codes;
  a.tags = tags;
  a.acodes = acodes;
  a.hcodes = hcodes;
  a.plane = nt * (int64_t)p->K * p->token_tile;
  a.bit_hist = bit_hist;
  a.rows = p->rows;
  a.K = p->K;
  a.T = p->token_tile;
  a.base = p->base;
  a.inv_base = (float)(1.0 / (double)p->base);
  a.base_dev = base_dev;
  a.k0 = p->thr0_log2;
  return launch_quantize(a, (hipStream_t)stream);
}

int linear_impl(const dstar_fmdq_params* p, const float* base_dev, int32_t N, const int8_t* codes,
                const uint16_t* perm, const int32_t* group_off, const int8_t* acodes,
                const int8_t* hcodes, const int8_t* w, const int8_t* w_t, const float* w_scale,
                const float* y_prev, float* y_out, float* gelu_out, int32_t* acc_dbg,
                int64_t* s_dbg, int32_t dbg_tile_lo, int32_t dbg_tile_hi, void* stream);

// Checks the device base pointer of the _dyn entry points.
int check_base_dev(const float* base_dev, const char* what) {
  if (base_dev == nullptr) return set_error(DSTAR_ENULL, "%s: base must not be NULL", what);
  if (!aligned(base_dev, 4)) return set_error(DSTAR_EALIGN, "%s: base must be 4-byte aligned", what);
  return DSTAR_OK;
}

}  // namespace

extern "C" {

int dstar_fmdq_quantize(const dstar_fmdq_params* p, const float* x_t, const float* x_prev,
                        int8_t* codes, uint8_t* tags, int8_t* acodes, int8_t* hcodes,
                        uint32_t* bit_hist, void* stream) {
  return quantize_impl(p, nullptr, x_t, x_prev, codes, tags, acodes, hcodes, bit_hist, stream);
}

int dstar_fmdq_quantize_dyn(const dstar_fmdq_params* p, const float* base, const float* x_t,
                            const float* x_prev, int8_t* codes, uint8_t* tags, int8_t* acodes,
                            int8_t* hcodes, uint32_t* bit_hist, void* stream) {
  clear_error();
  if (int rc = check_base_dev(base, "quantize_dyn")) return rc;
  return quantize_impl(p, base, x_t, x_prev, codes, tags, acodes, hcodes, bit_hist, stream);
}

int dstar_fmdq_dynamic_base(const dstar_fmdq_params* p, const float* x_t, const float* x_prev,
                            float* base, void* stream) {
  clear_error();
  int64_t nt = 0;
  if (int rc = check_params(p, &nt)) return rc;
  if (!base || (p->rows > 0 && (!x_t || !x_prev)))
    return set_error(DSTAR_ENULL, "dynamic_base: x_t, x_prev and base must not be NULL");
  if (!aligned(base, 4) || (p->rows > 0 && (!aligned(x_t, 16) || !aligned(x_prev, 16))))
    return set_error(DSTAR_EALIGN,
                     "dynamic_base: x_t and x_prev must be 16-byte aligned, base 4-byte aligned");
  BaseArgs a;
  a.x_t = x_t;
  a.x_prev = x_prev;
  a.base_bits = reinterpret_cast<uint32_t*>(base);
  a.rows = p->rows;
  a.K = p->K;
  a.T = p->token_tile;
  a.fallback = p->base;
  return launch_dynamic_base(a, (hipStream_t)stream);
}

int dstar_fmdq_bucket(const dstar_fmdq_params* p, const uint8_t* tags, uint16_t* perm,
                      int32_t* group_off, void* stream) {
  clear_error();
  int64_t nt = 0;
  if (int rc = check_params(p, &nt)) return rc;
  if (nt == 0) return DSTAR_OK;
  if (!tags || !perm || !group_off)
    return set_error(DSTAR_ENULL, "bucket: tags, perm and group_off must not be NULL");
  if (!aligned(perm, 2) || !aligned(group_off, 4))
    return set_error(DSTAR_EALIGN, "bucket: perm must be 2-byte and group_off 4-byte aligned");
  BucketArgs a;
  a.tags = tags;
  a.perm = perm;
  a.group_off = group_off;
  a.n_tiles = nt;
  a.K = p->K;
  return launch_bucket(a, (hipStream_t)stream);
}

int dstar_fmdq_slice_encode(const dstar_fmdq_params* p, const int8_t* codes, const uint8_t* tags,
                            uint32_t* entries, uint8_t* slices, int32_t* slice_off, void* stream) {
  clear_error();
  int64_t nt = 0;
  if (int rc = check_params(p, &nt)) return rc;
  if (p->K > DSTAR_FMDQ_SLICE_MAX_K)
    return set_error(DSTAR_EUNSUPPORTED, "slice_encode: K = %d above %d", p->K, DSTAR_FMDQ_SLICE_MAX_K);
  if (nt == 0) return DSTAR_OK;
  if (!codes || !tags || !entries || !slices || !slice_off)
    return set_error(DSTAR_ENULL, "slice_encode: codes, tags, entries, slices and slice_off must not be NULL");
  if (!aligned(codes, 16) || !aligned(entries, 4) || !aligned(slice_off, 4))
    return set_error(DSTAR_EALIGN, "slice_encode: codes must be 16-byte aligned, entries and slice_off 4-byte");
  SliceArgs a;
  a.codes = codes;
  a.tags = tags;
  a.entries = entries;
  a.slices = slices;
  a.slice_off = slice_off;
  a.n_tiles = nt;
  a.K = p->K;
  a.T = p->token_tile;
  return launch_slices(a, (hipStream_t)stream);
}

int dstar_fmdq_pack_weights(int32_t K, int32_t N, const int8_t* w, int8_t* w_t, void* stream) {
  clear_error();
  if (K < 1 || K > DSTAR_FMDQ_MAX_K)
    return set_error(DSTAR_EINVAL, "pack_weights: K = %d outside [1, %d]", K, DSTAR_FMDQ_MAX_K);
  if (N < 1 || N > (1 << 20))
    return set_error(DSTAR_EINVAL, "pack_weights: N = %d outside [1, 2^20]", N);
  if (!w || !w_t) return set_error(DSTAR_ENULL, "pack_weights: w and w_t must not be NULL");
  if (!aligned(w, 16) || !aligned(w_t, 16))
    return set_error(DSTAR_EALIGN, "pack_weights: w and w_t must be 16-byte aligned");
  return launch_pack_weights(K, N, w, w_t, (hipStream_t)stream);
}

int dstar_fmdq_linear(const dstar_fmdq_params* p, int32_t N, const int8_t* codes,
                      const uint16_t* perm, const int32_t* group_off,
                      const int8_t* acodes, const int8_t* hcodes, const int8_t* w,
                      const int8_t* w_t,
                      const float* w_scale, const float* y_prev, float* y_out, int32_t* acc_dbg,
                      int64_t* s_dbg, int32_t dbg_tile_lo, int32_t dbg_tile_hi, void* stream) {
  clear_error();
  return linear_impl(p, nullptr, N, codes, perm, group_off, acodes, hcodes, w, w_t, w_scale, y_prev,
                     y_out, nullptr, acc_dbg, s_dbg, dbg_tile_lo, dbg_tile_hi, stream);
}

int dstar_fmdq_linear_gelu(const dstar_fmdq_params* p, int32_t N, const int8_t* codes,
                           const uint16_t* perm, const int32_t* group_off, const int8_t* acodes,
                           const int8_t* hcodes, const int8_t* w, const int8_t* w_t,
                           const float* w_scale, const float* y_prev, float* y_out,
                           float* gelu_out, void* stream) {
  clear_error();
  if (gelu_out == nullptr) return set_error(DSTAR_ENULL, "linear_gelu: gelu_out must not be NULL");
  if (!aligned(gelu_out, 16)) return set_error(DSTAR_EALIGN, "linear_gelu: gelu_out must be 16-byte aligned");
  // Workgroups read Y_{t-1} and write Y_t and GELU(Y_t) of their own block
  // only, so gelu_out may not share a byte with either (not even shifted by a
  // row: another block's GELU store would race with this block's loads).
  if (p != nullptr && p->rows > 0 && N > 0) {
    const uintptr_t bytes = (uintptr_t)p->rows * (uintptr_t)N * sizeof(float);
    auto overlap = [bytes](const void* x, const void* y) {
      const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
      return x != nullptr && y != nullptr && a < b + bytes && b < a + bytes;
    };
    if (overlap(gelu_out, y_out) || overlap(gelu_out, y_prev))
      return set_error(DSTAR_EINVAL, "linear_gelu: gelu_out overlaps y_prev or y_out");
  }
  return linear_impl(p, nullptr, N, codes, perm, group_off, acodes, hcodes, w, w_t, w_scale, y_prev,
                     y_out, gelu_out, nullptr, nullptr, 0, 0, stream);
}

int dstar_fmdq_gelu(const float* y, float* g, int64_t n, void* stream) {
  clear_error();
  if (n < 0) return set_error(DSTAR_EINVAL, "gelu: n = %lld < 0", (long long)n);
  if (n == 0) return DSTAR_OK;
  if (!y || !g) return set_error(DSTAR_ENULL, "gelu: y and g must not be NULL");
  if (!aligned(y, 16) || !aligned(g, 16)) return set_error(DSTAR_EALIGN, "gelu: y and g must be 16-byte aligned");
  return launch_gelu(y, g, n, (hipStream_t)stream);
}

int dstar_fmdq_linear_dyn(const dstar_fmdq_params* p, const float* base, int32_t N,
                          const int8_t* codes, const uint16_t* perm, const int32_t* group_off,
                          const int8_t* acodes, const int8_t* hcodes, const int8_t* w,
                          const int8_t* w_t, const float* w_scale, const float* y_prev,
                          float* y_out, int32_t* acc_dbg, int64_t* s_dbg, int32_t dbg_tile_lo,
                          int32_t dbg_tile_hi, void* stream) {
  clear_error();
  if (int rc = check_base_dev(base, "linear_dyn")) return rc;
  return linear_impl(p, base, N, codes, perm, group_off, acodes, hcodes, w, w_t, w_scale, y_prev,
                     y_out, nullptr, acc_dbg, s_dbg, dbg_tile_lo, dbg_tile_hi, stream);
}

}  // extern "C"

namespace {

int linear_impl(const dstar_fmdq_params* p, const float* base_dev, int32_t N, const int8_t* codes,
                const uint16_t* perm, const int32_t* group_off, const int8_t* acodes,
                const int8_t* hcodes, const int8_t* w, const int8_t* w_t, const float* w_scale,
                const float* y_prev, float* y_out, float* gelu_out, int32_t* acc_dbg,
                int64_t* s_dbg, int32_t dbg_tile_lo, int32_t dbg_tile_hi, void* stream) {
  int64_t nt = 0;
  if (int rc = check_params(p, &nt)) return rc;
  if (N < 1 || N > (1 << 20) || N % 4 != 0)
    return set_error(DSTAR_EINVAL, "linear: N = %d must be a multiple of 4 in [4, 2^20]", N);
  if ((acc_dbg || s_dbg) && (dbg_tile_lo < 0 || dbg_tile_lo >= dbg_tile_hi || dbg_tile_hi > nt))
    return set_error(DSTAR_EINVAL, "linear: debug tile range [%d, %d) not within [0, %lld)",
                     dbg_tile_lo, dbg_tile_hi, (long long)nt);
  if (nt == 0) return DSTAR_OK;
  if (!perm || !group_off || !w || !w_scale || !y_prev || !y_out)
    return set_error(DSTAR_ENULL,
                     "linear: perm, group_off, w, w_scale, y_prev and y_out must not be NULL");
  if (!codes && (!acodes || !hcodes))
    return set_error(DSTAR_ENULL, "linear: codes may be NULL only when acodes and hcodes are given");
  if ((codes && !aligned(codes, 16)) || !aligned(w, 16) || !aligned(y_prev, 16) || !aligned(y_out, 16) ||
      !aligned(w_scale, 4) || !aligned(perm, 2) || !aligned(group_off, 4) ||
      (acc_dbg && !aligned(acc_dbg, 4)) || (s_dbg && !aligned(s_dbg, 8)) ||
      (acodes && !aligned(acodes, 16)) ||
      (hcodes && !aligned(hcodes, 16)) || (w_t && !aligned(w_t, 16)))
    return set_error(DSTAR_EALIGN,
                     "linear: codes, acodes, hcodes, w, w_t, y_prev, y_out must be 16-byte aligned "
                     "(s_dbg 8-byte, w_scale, group_off, acc_dbg 4-byte, perm 2-byte)");
  LinearArgs a;
  a.codes = codes;
  a.perm = perm;
  a.group_off = group_off;
  a.acodes = acodes;
  a.hcodes = hcodes;
  a.w = w;
  a.w_t = w_t;
  a.w_scale = w_scale;
  a.y_prev = y_prev;
  a.y_out = y_out;
  a.acc_dbg = acc_dbg;
  a.s_dbg = s_dbg;
  a.dbg_lo = dbg_tile_lo;
  a.dbg_hi = dbg_tile_hi;
  a.rows = p->rows;
  a.K = p->K;
  a.N = N;
  a.T = p->token_tile;
  a.base = (double)p->base;
  a.base_dev = base_dev;
  a.gelu_out = gelu_out;
  return launch_linear(a, (hipStream_t)stream);
}

}  // namespace

// ---------------------------------------------------------------------------
// The whole layer in one call, with the intermediates in a caller workspace.

namespace dstar {

namespace {
inline int64_t round256(int64_t v) { return (v + 255) & ~int64_t(255); }
}  // namespace

LayerWorkspace layer_workspace(int64_t nt, int64_t K, int64_t T) {
  LayerWorkspace w;
  int64_t o = 0;
  w.codes = o;  o += round256(nt * K * T);
  w.acodes = o; o += round256(nt * T * K);
  w.hcodes = o; o += round256(2 * nt * K * T);
  w.tags = o;   o += round256(nt * K);
  w.perm = o;   o += round256(2 * nt * K);
  w.off = o;    o += round256(4 * nt * (DSTAR_FMDQ_NUM_BINS + 1));
  w.total = o;
  return w;
}

int layer_impl(const dstar_fmdq_params* p, int32_t N, const float* x_t, const float* x_prev,
               const int8_t* w, const int8_t* w_t, const float* w_scale, const float* y_prev,
               float* y_out, uint32_t* bit_hist, void* workspace, int64_t workspace_bytes,
               void* stream) {
  int64_t nt = 0;
  if (int rc = check_params(p, &nt)) return rc;
  if (N < 1 || N > (1 << 20) || N % 4 != 0)
    return set_error(DSTAR_EINVAL, "layer: N = %d must be a multiple of 4 in [4, 2^20]", N);
  if (nt == 0) return DSTAR_OK;
  const LayerWorkspace ws = layer_workspace(nt, p->K, p->token_tile);
  if (workspace == nullptr) return set_error(DSTAR_ENULL, "layer: workspace must not be NULL");
  if (!aligned(workspace, 256)) return set_error(DSTAR_EALIGN, "layer: workspace must be 256-byte aligned");
  if (workspace_bytes < ws.total)
    return set_error(DSTAR_EINVAL, "layer: workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                     (long long)ws.total);
  uint8_t* b = static_cast<uint8_t*>(workspace);
  int8_t* codes = reinterpret_cast<int8_t*>(b + ws.codes);
  int8_t* acodes = reinterpret_cast<int8_t*>(b + ws.acodes);
  int8_t* hcodes = reinterpret_cast<int8_t*>(b + ws.hcodes);
  uint8_t* tags = b + ws.tags;
  uint16_t* perm = reinterpret_cast<uint16_t*>(b + ws.perm);
  int32_t* off = reinterpret_cast<int32_t*>(b + ws.off);
  if (int rc = quantize_impl(p, nullptr, x_t, x_prev, codes, tags, acodes, hcodes, bit_hist, stream)) return rc;
  if (int rc = dstar_fmdq_bucket(p, tags, perm, off, stream)) return rc;
  return linear_impl(p, nullptr, N, codes, perm, off, acodes, hcodes, w, w_t, w_scale, y_prev, y_out, nullptr,
                     nullptr, nullptr, 0, 0, stream);
}

}  // namespace dstar

extern "C" {

int64_t dstar_fmdq_layer_workspace_size(const dstar_fmdq_params* p) {
  clear_error();
  int64_t nt = 0;
  if (int rc = check_params(p, &nt)) return rc;
  return layer_workspace(nt, p->K, p->token_tile).total;
}

int dstar_fmdq_layer(const dstar_fmdq_params* p, int32_t N, const float* x_t, const float* x_prev,
                     const int8_t* w, const int8_t* w_t, const float* w_scale, const float* y_prev,
                     float* y_out, uint32_t* bit_hist, void* workspace, int64_t workspace_bytes,
                     void* stream) {
  clear_error();
  return layer_impl(p, N, x_t, x_prev, w, w_t, w_scale, y_prev, y_out, bit_hist, workspace,
                    workspace_bytes, stream);
}

}  // extern "C"
