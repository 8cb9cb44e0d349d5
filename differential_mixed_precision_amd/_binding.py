"""ctypes binding of libdstar_fmdq.so (the C ABI declared in include/dstar_fmdq.h
and include/dstar_sar.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library.  Tensors are torch tensors on the GPU (their data_ptr() is passed
through); torch is used for device memory and streams, nothing else.  If the
library has not been built, every call raises — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# DSTAR_FMDQ_LIB names another build of the same library (the host-sanitized
# one); by default the in-tree build next to this file is loaded.
LIB_PATH = os.environ.get("DSTAR_FMDQ_LIB") or os.path.join(_PKG, "libdstar_fmdq.so")

OK, EINVAL, ENULL, EALIGN, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4, -5
NUM_TAGS = 16
NUM_BINS = 64
TAG_OFFSET = 15
POT_MAX = 21
PREC_SHIFT = 4
MAX_K = 65535
ABI_VERSION = 10
SAR_BLOCK = 64
SAR_TILE = 32
SAR_PAD = 32
SAR_MAX_D = 128
SAR_MAX_L = 65536
SAR_EXP_FRAC = 36
NOALLOC_MAX_BYTES = 64 << 20

SYMBOLS = ("dstar_fmdq_quantize", "dstar_fmdq_bucket", "dstar_fmdq_slice_encode", "dstar_fmdq_pack_weights",
           "dstar_fmdq_linear", "dstar_fmdq_linear_gelu", "dstar_fmdq_gelu",
           "dstar_fmdq_dynamic_base", "dstar_fmdq_quantize_dyn",
           "dstar_fmdq_linear_dyn", "dstar_fmdq_layer", "dstar_fmdq_layer_workspace_size",
           "dstar_fmdq_layer_noalloc",
           "dstar_fmdq_last_error", "dstar_fmdq_abi_version")
SAR_SYMBOLS = ("dstar_sar_quantize_q", "dstar_sar_quantize_k", "dstar_sar_quantize_v", "dstar_sar_scores",
               "dstar_sar_pv")


class FmdqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dstar_fmdq error {code}: {msg}")
        self.code = code


class Params(ctypes.Structure):
    """dstar_fmdq_params."""
    _fields_ = [("rows", ctypes.c_int32), ("tokens_per_seq", ctypes.c_int32),
                ("K", ctypes.c_int32), ("token_tile", ctypes.c_int32),
                ("base", ctypes.c_float), ("thr0_log2", ctypes.c_int32)]


class SarParams(ctypes.Structure):
    """dstar_sar_params."""
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("tokens", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("base_q", ctypes.c_float), ("base_p", ctypes.c_float),
                ("sm_scale", ctypes.c_float)]


_lib = None


def load() -> ctypes.CDLL:
    """Loads the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m differential_mixed_precision_amd.build` "
            "(or __graft_entry__.build()).  There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Params)
    vp = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.dstar_fmdq_quantize.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.dstar_fmdq_quantize.restype = ctypes.c_int
    lib.dstar_fmdq_bucket.argtypes = [P, vp, vp, vp, vp]
    lib.dstar_fmdq_bucket.restype = ctypes.c_int
    lib.dstar_fmdq_slice_encode.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.dstar_fmdq_slice_encode.restype = ctypes.c_int
    lib.dstar_fmdq_pack_weights.argtypes = [i32, i32, vp, vp, vp]
    lib.dstar_fmdq_pack_weights.restype = ctypes.c_int
    lib.dstar_fmdq_linear.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp]
    lib.dstar_fmdq_linear.restype = ctypes.c_int
    lib.dstar_fmdq_linear_gelu.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.dstar_fmdq_linear_gelu.restype = ctypes.c_int
    lib.dstar_fmdq_gelu.argtypes = [vp, vp, ctypes.c_int64, vp]
    lib.dstar_fmdq_gelu.restype = ctypes.c_int
    lib.dstar_fmdq_dynamic_base.argtypes = [P, vp, vp, vp, vp]
    lib.dstar_fmdq_dynamic_base.restype = ctypes.c_int
    lib.dstar_fmdq_quantize_dyn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.dstar_fmdq_quantize_dyn.restype = ctypes.c_int
    lib.dstar_fmdq_linear_dyn.argtypes = [P, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          i32, i32, vp]
    lib.dstar_fmdq_linear_dyn.restype = ctypes.c_int
    lib.dstar_fmdq_layer.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp]
    lib.dstar_fmdq_layer.restype = ctypes.c_int
    lib.dstar_fmdq_layer_noalloc.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.dstar_fmdq_layer_noalloc.restype = ctypes.c_int
    lib.dstar_fmdq_layer_workspace_size.argtypes = [P]
    lib.dstar_fmdq_layer_workspace_size.restype = ctypes.c_int64
    S = ctypes.POINTER(SarParams)
    lib.dstar_sar_quantize_q.argtypes = [S, vp, vp, vp, vp]
    lib.dstar_sar_quantize_k.argtypes = [S, vp, vp, vp, vp]
    lib.dstar_sar_quantize_v.argtypes = [S, vp, vp, vp, vp]
    lib.dstar_sar_scores.argtypes = [S, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.dstar_sar_pv.argtypes = [S, vp, vp, i32, vp, vp, vp, vp, vp, vp]
    for name in SAR_SYMBOLS:
        getattr(lib, name).restype = ctypes.c_int
    lib.dstar_fmdq_last_error.argtypes = []
    lib.dstar_fmdq_last_error.restype = ctypes.c_char_p
    lib.dstar_fmdq_abi_version.argtypes = []
    lib.dstar_fmdq_abi_version.restype = ctypes.c_int
    if lib.dstar_fmdq_abi_version() != ABI_VERSION:
        raise RuntimeError("libdstar_fmdq.so ABI version mismatch; rebuild it")
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int) -> None:
    if rc != OK:
        raise FmdqError(rc, load().dstar_fmdq_last_error().decode())


def make_params(rows: int, K: int, token_tile: int, base: float, thr0_log2: int,
                tokens_per_seq: int | None = None) -> Params:
    return Params(int(rows), int(rows if tokens_per_seq is None else tokens_per_seq), int(K),
                  int(token_tile), float(base), int(thr0_log2))


def quantize(p: Params, x_t, x_prev, codes, tags, acodes=None, hcodes=None, bit_hist=None,
             stream=None) -> None:
    """dstar_fmdq_quantize."""
    _check(load().dstar_fmdq_quantize(ctypes.byref(p), _ptr(x_t), _ptr(x_prev), _ptr(codes),
                                      _ptr(tags), _ptr(acodes), _ptr(hcodes), _ptr(bit_hist),
                                      _stream(stream)))


def bucket(p: Params, tags, perm, group_off, stream=None) -> None:
    """dstar_fmdq_bucket."""
    _check(load().dstar_fmdq_bucket(ctypes.byref(p), _ptr(tags), _ptr(perm), _ptr(group_off),
                                    _stream(stream)))


def pack_weights(K: int, N: int, w, w_t, stream=None) -> None:
    """dstar_fmdq_pack_weights: w_t[n][k] = w[k][n]."""
    _check(load().dstar_fmdq_pack_weights(int(K), int(N), _ptr(w), _ptr(w_t), _stream(stream)))


def linear(p: Params, N: int, codes, perm, group_off, acodes, hcodes, w, w_t, w_scale, y_prev,
           y_out, acc_dbg=None, dbg_tile_lo: int = 0, dbg_tile_hi: int = 0, stream=None,
           s_dbg=None) -> None:
    """dstar_fmdq_linear."""
    _check(load().dstar_fmdq_linear(ctypes.byref(p), int(N), _ptr(codes), _ptr(perm),
                                    _ptr(group_off), _ptr(acodes), _ptr(hcodes), _ptr(w), _ptr(w_t),
                                    _ptr(w_scale), _ptr(y_prev), _ptr(y_out), _ptr(acc_dbg),
                                    _ptr(s_dbg), int(dbg_tile_lo), int(dbg_tile_hi), _stream(stream)))


def layer_workspace_size(p: Params) -> int:
    """dstar_fmdq_layer_workspace_size: bytes of workspace the one-call layer needs."""
    n = load().dstar_fmdq_layer_workspace_size(ctypes.byref(p))
    if n < 0:
        _check(int(n))
    return int(n)


def layer(p: Params, N: int, x_t, x_prev, w, w_t, w_scale, y_prev, y_out, workspace, bit_hist=None,
          stream=None) -> None:
    """dstar_fmdq_layer: the three stages in one call; ``workspace`` is a uint8
    device tensor of at least layer_workspace_size(p) bytes."""
    _check(load().dstar_fmdq_layer(ctypes.byref(p), int(N), _ptr(x_t), _ptr(x_prev), _ptr(w), _ptr(w_t),
                                   _ptr(w_scale), _ptr(y_prev), _ptr(y_out), _ptr(bit_hist), _ptr(workspace),
                                   int(workspace.numel() * workspace.element_size()), _stream(stream)))


def layer_noalloc(p: Params, N: int, x_t, x_prev, w, w_t, w_scale, y_prev, y_out, bit_hist=None,
                  stream=None) -> None:
    """dstar_fmdq_layer_noalloc: the three stages in one call with the
    intermediates in the library's own per-GPU scratch (at most
    NOALLOC_MAX_BYTES of them; calls that overlap in time on one GPU race)."""
    _check(load().dstar_fmdq_layer_noalloc(ctypes.byref(p), int(N), _ptr(x_t), _ptr(x_prev), _ptr(w), _ptr(w_t),
                                           _ptr(w_scale), _ptr(y_prev), _ptr(y_out), _ptr(bit_hist),
                                           _stream(stream)))


def dynamic_base(p: Params, x_t, x_prev, base, stream=None) -> None:
    """dstar_fmdq_dynamic_base: base (a 1-element float32 device tensor) = the
    smallest positive sub-channel maximum of |x_t - x_prev|."""
    _check(load().dstar_fmdq_dynamic_base(ctypes.byref(p), _ptr(x_t), _ptr(x_prev), _ptr(base),
                                          _stream(stream)))


def quantize_dyn(p: Params, base, x_t, x_prev, codes, tags, acodes=None, hcodes=None, bit_hist=None,
                 stream=None) -> None:
    """dstar_fmdq_quantize_dyn: stage 1 with the base read from the device tensor `base`."""
    _check(load().dstar_fmdq_quantize_dyn(ctypes.byref(p), _ptr(base), _ptr(x_t), _ptr(x_prev),
                                          _ptr(codes), _ptr(tags), _ptr(acodes), _ptr(hcodes),
                                          _ptr(bit_hist), _stream(stream)))


def linear_dyn(p: Params, base, N: int, codes, perm, group_off, acodes, hcodes, w, w_t, w_scale,
               y_prev, y_out, acc_dbg=None, dbg_tile_lo: int = 0, dbg_tile_hi: int = 0,
               stream=None, s_dbg=None) -> None:
    """dstar_fmdq_linear_dyn: stage 3 with the base read from the device tensor `base`."""
    _check(load().dstar_fmdq_linear_dyn(ctypes.byref(p), _ptr(base), int(N), _ptr(codes), _ptr(perm),
                                        _ptr(group_off), _ptr(acodes), _ptr(hcodes), _ptr(w),
                                        _ptr(w_t), _ptr(w_scale), _ptr(y_prev), _ptr(y_out),
                                        _ptr(acc_dbg), _ptr(s_dbg), int(dbg_tile_lo), int(dbg_tile_hi),
                                        _stream(stream)))


def linear_gelu(p: Params, N: int, codes, perm, group_off, acodes, hcodes, w, w_t, w_scale, y_prev,
                y_out, gelu_out, stream=None) -> None:
    """dstar_fmdq_linear_gelu: stage 3 that also stores GELU(Y_t) in gelu_out."""
    _check(load().dstar_fmdq_linear_gelu(ctypes.byref(p), int(N), _ptr(codes), _ptr(perm),
                                         _ptr(group_off), _ptr(acodes), _ptr(hcodes), _ptr(w),
                                         _ptr(w_t), _ptr(w_scale), _ptr(y_prev), _ptr(y_out),
                                         _ptr(gelu_out), _stream(stream)))


def gelu(y, g, n: int | None = None, stream=None) -> None:
    """dstar_fmdq_gelu: g = GELU(y) elementwise (n defaults to y.numel())."""
    _check(load().dstar_fmdq_gelu(_ptr(y), _ptr(g), int(y.numel() if n is None else n), _stream(stream)))


def slice_encode(p: Params, codes, tags, entries, slices, slice_off, stream=None) -> None:
    """dstar_fmdq_slice_encode: the 2-bit slice stream of every token tile."""
    _check(load().dstar_fmdq_slice_encode(ctypes.byref(p), _ptr(codes), _ptr(tags), _ptr(entries),
                                          _ptr(slices), _ptr(slice_off), _stream(stream)))


# ---------------------------------------------------------------- SAR attention

def sar_padded_dim(d: int) -> int:
    """dp = d rounded up to a multiple of SAR_PAD (the codes' row length)."""
    return (int(d) + SAR_PAD - 1) // SAR_PAD * SAR_PAD


def make_sar_params(batch: int, heads: int, tokens: int, head_dim: int, base_q: float, base_p: float,
                    sm_scale: float) -> SarParams:
    return SarParams(int(batch), int(heads), int(tokens), int(head_dim), float(base_q), float(base_p),
                     float(sm_scale))


def sar_quantize_q(p: SarParams, q, qcodes, qpot, stream=None) -> None:
    """dstar_sar_quantize_q."""
    _check(load().dstar_sar_quantize_q(ctypes.byref(p), _ptr(q), _ptr(qcodes), _ptr(qpot), _stream(stream)))


def sar_quantize_k(p: SarParams, k, kcodes, kscale, stream=None) -> None:
    """dstar_sar_quantize_k."""
    _check(load().dstar_sar_quantize_k(ctypes.byref(p), _ptr(k), _ptr(kcodes), _ptr(kscale), _stream(stream)))


def sar_quantize_v(p: SarParams, v, vcodes_t, vscale, stream=None) -> None:
    """dstar_sar_quantize_v."""
    _check(load().dstar_sar_quantize_v(ctypes.byref(p), _ptr(v), _ptr(vcodes_t), _ptr(vscale), _stream(stream)))


def sar_scores(p: SarParams, row_ptr, cols, nnz: int, qcodes, qpot, kcodes, kscale, pcodes, ppot,
               stream=None) -> None:
    """dstar_sar_scores."""
    _check(load().dstar_sar_scores(ctypes.byref(p), _ptr(row_ptr), _ptr(cols), int(nnz), _ptr(qcodes),
                                   _ptr(qpot), _ptr(kcodes), _ptr(kscale), _ptr(pcodes), _ptr(ppot),
                                   _stream(stream)))


def sar_pv(p: SarParams, row_ptr, cols, nnz: int, pcodes, ppot, vcodes_t, vscale, out, stream=None) -> None:
    """dstar_sar_pv."""
    _check(load().dstar_sar_pv(ctypes.byref(p), _ptr(row_ptr), _ptr(cols), int(nnz), _ptr(pcodes), _ptr(ppot),
                               _ptr(vcodes_t), _ptr(vscale), _ptr(out), _stream(stream)))
