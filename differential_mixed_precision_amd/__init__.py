"""FMDQ differential linear layer (DSTAR, arXiv 2607.15846) on AMD MI355X.

The layer runs in three HIP kernels behind a C ABI (include/dstar_fmdq.h):
``quantize`` (differential + sub-channel quantization), ``bucket`` (reorder
channels by FPoT tag) and ``linear`` (grouped int8 GEMM with shift alignment,
dequantization and the reverse differential).  ``dynamic_base`` with
``quantize_dyn`` / ``linear_dyn`` is the variant whose base is the smallest
sub-channel maximum of the data instead of a static one.  This package is the
thin Python binding; ``FmdqLayer`` allocates the buffers of one layer with
torch and calls the stages on the current stream.
"""
from __future__ import annotations

from . import _binding
from ._binding import (FmdqError, Params, bucket, dynamic_base, linear, linear_dyn,  # noqa: F401
                       load, make_params, pack_weights, quantize, quantize_dyn)

__all__ = ["FmdqError", "Params", "FmdqLayer", "bucket", "dynamic_base", "linear", "linear_dyn",
           "load", "make_params", "pack_weights", "quantize", "quantize_dyn", "n_tiles"]


def n_tiles(rows: int, token_tile: int) -> int:
    return (rows + token_tile - 1) // token_tile


class FmdqLayer:
    """Device buffers of one FMDQ differential linear layer and its three calls.

    ``step(x_t, x_prev, y)`` updates the cached output ``y`` in place:
    y ← y + w_scale · W · Δ̂, with Δ̂ the FMDQ-quantized X_t − X_{t−1}.
    ``step_dynamic`` does the same with the dynamic base (one more pass over
    X first); the base it used is left in ``self.base_dev``.
    """

    def __init__(self, w, w_scale, rows: int, token_tile: int, base: float, thr0_log2: int,
                 tokens_per_seq: int | None = None):
        import torch
        assert w.dtype == torch.int8 and w.is_cuda and w.dim() == 2
        self.K, self.N = int(w.shape[0]), int(w.shape[1])
        self.w, self.w_scale = w.contiguous(), w_scale.contiguous()
        self.p = make_params(rows, self.K, token_tile, base, thr0_log2, tokens_per_seq)
        self.T = token_tile
        nt = n_tiles(rows, token_tile)
        dev = w.device
        self.codes = torch.empty((nt, self.K, token_tile), dtype=torch.int8, device=dev)
        self.tags = torch.empty((nt, self.K), dtype=torch.uint8, device=dev)
        self.acodes = torch.empty((nt * token_tile, self.K), dtype=torch.int8, device=dev)
        self.hcodes = torch.empty((2, nt, self.K, token_tile), dtype=torch.int8, device=dev)
        self.w_t = torch.empty((self.N, self.K), dtype=torch.int8, device=dev)
        pack_weights(self.K, self.N, self.w, self.w_t)
        self.perm = torch.empty((nt, self.K), dtype=torch.int16, device=dev)  # uint16 ids
        self.group_off = torch.empty((nt, 65), dtype=torch.int32, device=dev)
        self.bit_hist = torch.zeros(4, dtype=torch.int32, device=dev)
        self.base_dev = torch.empty(1, dtype=torch.float32, device=dev)

    def step(self, x_t, x_prev, y, y_out=None, stream=None, hist: bool = True):
        quantize(self.p, x_t, x_prev, self.codes, self.tags, self.acodes, self.hcodes,
                 self.bit_hist if hist else None, stream)
        bucket(self.p, self.tags, self.perm, self.group_off, stream)
        out = y if y_out is None else y_out
        linear(self.p, self.N, self.codes, self.perm, self.group_off, self.acodes, self.hcodes,
               self.w, self.w_t, self.w_scale, y, out, stream=stream)
        return out

    def step_dynamic(self, x_t, x_prev, y, y_out=None, stream=None, hist: bool = True):
        dynamic_base(self.p, x_t, x_prev, self.base_dev, stream)
        quantize_dyn(self.p, self.base_dev, x_t, x_prev, self.codes, self.tags, self.acodes,
                     self.hcodes, self.bit_hist if hist else None, stream)
        bucket(self.p, self.tags, self.perm, self.group_off, stream)
        out = y if y_out is None else y_out
        linear_dyn(self.p, self.base_dev, self.N, self.codes, self.perm, self.group_off, self.acodes,
                   self.hcodes, self.w, self.w_t, self.w_scale, y, out, stream=stream)
        return out
