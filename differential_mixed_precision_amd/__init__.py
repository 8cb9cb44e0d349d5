"""FMDQ differential linear layer (DSTAR, arXiv 2607.15846) on AMD MI355X.

The layer runs in three HIP kernels behind a C ABI (include/dstar_fmdq.h):
``quantize`` (differential + sub-channel quantization), ``bucket`` (reorder
channels by FPoT tag) and ``linear`` (grouped int8 GEMM with shift alignment,
dequantization and the reverse differential).  ``dynamic_base`` with
``quantize_dyn`` / ``linear_dyn`` is the variant whose base is the smallest
sub-channel maximum of the data instead of a static one; ``linear_gelu`` fuses
the MLP's GELU into stage 3 and ``gelu`` is the same activation on its own.
This package is the thin Python binding; ``FmdqLayer`` allocates the buffers of
one layer with torch and calls the stages on the current stream, and
``FmdqMLP`` chains two of them (fc1 → GELU → fc2) over timesteps.

``SarAttention`` is Sparse Attention Reuse with FMDQ-INT8 operands (DSTAR
§3.2, §4.3; include/dstar_sar.h): a cached step that quantizes Q, K and V and
stores the block-sparse attention weights, and reused steps that apply them to
the current V.
"""
from __future__ import annotations

from . import _binding
from ._binding import (FmdqError, Params, bucket, dynamic_base, gelu, layer, layer_noalloc,  # noqa: F401
                       layer_workspace_size,
                       linear, linear_dyn, linear_gelu, load, make_params, pack_weights, quantize,
                       quantize_dyn, slice_encode, sar_padded_dim, sar_pv, sar_quantize_k,
                       sar_quantize_q, sar_quantize_v, sar_scores)

__all__ = ["FmdqError", "Params", "FmdqLayer", "FmdqMLP", "bucket", "dynamic_base", "gelu", "layer",
           "layer_noalloc", "layer_workspace_size", "linear",
           "linear_dyn", "linear_gelu", "load", "make_params", "pack_weights", "quantize",
           "quantize_dyn", "slice_encode", "n_tiles", "SarAttention", "sar_padded_dim", "sar_pv",
           "sar_quantize_k", "sar_quantize_q", "sar_quantize_v", "sar_scores"]


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
                 tokens_per_seq: int | None = None, plain_codes: bool = True):
        import torch
        assert w.dtype == torch.int8 and w.is_cuda and w.dim() == 2
        self.K, self.N = int(w.shape[0]), int(w.shape[1])
        self.w, self.w_scale = w.contiguous(), w_scale.contiguous()
        self.p = make_params(rows, self.K, token_tile, base, thr0_log2, tokens_per_seq)
        self.T = token_tile
        nt = n_tiles(rows, token_tile)
        dev = w.device
        # The plain codes ([n_t][K][T]) are read only by the per-group kernel
        # and the 2-bit slice stream; the MFMA kernels multiply the aligned
        # codes and digit planes, so with plain_codes=False stage 1 skips them.
        self.codes = (torch.empty((nt, self.K, token_tile), dtype=torch.int8, device=dev)
                      if plain_codes else None)
        self.tags = torch.empty((nt, self.K), dtype=torch.uint8, device=dev)
        self.acodes = torch.empty((nt * token_tile, self.K), dtype=torch.int8, device=dev)
        self.hcodes = torch.empty((2, nt, self.K, token_tile), dtype=torch.int8, device=dev)
        self.w_t = torch.empty((self.N, self.K), dtype=torch.int8, device=dev)
        pack_weights(self.K, self.N, self.w, self.w_t)
        self.perm = torch.empty((nt, self.K), dtype=torch.int16, device=dev)  # uint16 ids
        self.group_off = torch.empty((nt, 65), dtype=torch.int32, device=dev)
        self.bit_hist = torch.zeros(4, dtype=torch.int32, device=dev)
        self.base_dev = torch.empty(1, dtype=torch.float32, device=dev)

    def step(self, x_t, x_prev, y, y_out=None, stream=None, hist: bool = True, gelu_out=None):
        """One timestep pair; with ``gelu_out`` stage 3 also stores GELU(Y_t) there."""
        quantize(self.p, x_t, x_prev, self.codes, self.tags, self.acodes, self.hcodes,
                 self.bit_hist if hist else None, stream)
        bucket(self.p, self.tags, self.perm, self.group_off, stream)
        out = y if y_out is None else y_out
        if gelu_out is None:
            linear(self.p, self.N, self.codes, self.perm, self.group_off, self.acodes, self.hcodes,
                   self.w, self.w_t, self.w_scale, y, out, stream=stream)
        else:
            linear_gelu(self.p, self.N, self.codes, self.perm, self.group_off, self.acodes,
                        self.hcodes, self.w, self.w_t, self.w_scale, y, out, gelu_out, stream=stream)
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


class FmdqMLP:
    """The MLP of a DiT block, fc1 → GELU → fc2, run differentially over
    timesteps (DSTAR Eq. 1 for both linears; the GELU fused into fc1's stage 3
    as in DSTAR §4.3).

    State kept on the device between steps: Y1 (fc1's cached output, updated
    in place), G_t and G_{t−1} = GELU(Y1) at this and the previous step (two
    buffers used in turn; they are fc2's X_t and X_{t−1}) and Y2 (fc2's cached
    output, updated in place).  ``start(y1, y2)`` takes the cached outputs of
    the last full step and forms G from Y1; each ``step(x_t, x_prev)`` then
    runs fc1 with the fused GELU and fc2 on G_t − G_{t−1}.
    """

    def __init__(self, w1, ws1, base1: float, w2, ws2, base2: float, rows: int, token_tile: int,
                 thr0_log2: int, tokens_per_seq: int | None = None):
        import torch
        self.fc1 = FmdqLayer(w1, ws1, rows, token_tile, base1, thr0_log2, tokens_per_seq)
        self.fc2 = FmdqLayer(w2, ws2, rows, token_tile, base2, thr0_log2, tokens_per_seq)
        assert self.fc1.N == self.fc2.K
        self.g = [torch.empty((rows, self.fc1.N), dtype=torch.float32, device=w1.device) for _ in range(2)]
        self.cur = 0
        self.y1 = self.y2 = None

    def start(self, y1, y2, stream=None) -> None:
        self.y1, self.y2 = y1, y2
        self.cur = 0
        gelu(y1, self.g[0], stream=stream)

    @property
    def g_cur(self):
        """GELU(Y1) of the latest step (fc2's latest input)."""
        return self.g[self.cur]

    def step(self, x_t, x_prev, stream=None, hist: bool = True):
        nxt = 1 - self.cur
        self.fc1.step(x_t, x_prev, self.y1, stream=stream, hist=hist, gelu_out=self.g[nxt])
        self.fc2.step(self.g[nxt], self.g[self.cur], self.y2, stream=stream, hist=hist)
        self.cur = nxt
        return self.y2


class SarAttention:
    """One attention layer under Sparse Attention Reuse with FMDQ-INT8 operands
    (DSTAR §3.2 Fig. 8, §4.3 Fig. 13).

    ``mask`` is the static block mask, bool [heads][L/64][L/64] (numpy or
    torch); it is turned into compressed rows once, here.  Every buffer of the
    layer (codes, scales, the P cache, the output) is allocated once on
    ``device``.  ``cached_step(q, k, v)`` quantizes the three operands, fills the
    cache and returns O; ``reused_step(v)`` quantizes the current V and returns
    O = P_cache V.  q, k, v: float32 [batch·heads][L][d] on the device.
    """

    def __init__(self, mask, batch: int, heads: int, tokens: int, head_dim: int, base_q: float,
                 base_p: float, sm_scale: float, device="cuda"):
        import numpy as np
        import torch

        m = mask.cpu().numpy() if hasattr(mask, "cpu") else np.asarray(mask)
        nb = tokens // _binding.SAR_BLOCK
        if m.shape != (heads, nb, nb):
            raise ValueError(f"mask shape {m.shape} != {(heads, nb, nb)}")
        rows = m.astype(bool).reshape(heads * nb, nb)
        row_ptr = np.zeros(heads * nb + 1, dtype=np.int32)
        row_ptr[1:] = np.cumsum(rows.sum(axis=1))
        cols = np.nonzero(rows)[1].astype(np.int32)
        self.nnz = int(len(cols))
        self.p = _binding.make_sar_params(batch, heads, tokens, head_dim, base_q, base_p, sm_scale)
        dev = torch.device(device)
        BH, L, d = batch * heads, tokens, head_dim
        dp = sar_padded_dim(d)
        self.row_ptr = torch.from_numpy(row_ptr).to(dev)
        self.cols = torch.from_numpy(cols if len(cols) else np.zeros(1, np.int32)).to(dev)
        self.qcodes = torch.empty((BH, L, dp), dtype=torch.int8, device=dev)
        self.qpot = torch.empty((BH, L // _binding.SAR_TILE, dp), dtype=torch.uint8, device=dev)
        self.kcodes = torch.empty((BH, L, dp), dtype=torch.int8, device=dev)
        self.kscale = torch.empty((BH, L), dtype=torch.float32, device=dev)
        self.vcodes_t = torch.empty((BH, dp, L), dtype=torch.int8, device=dev)
        self.vscale = torch.empty((BH, d), dtype=torch.float32, device=dev)
        blocks = max(self.nnz, 1)
        self.pcodes = torch.empty((batch, blocks, 64, 64), dtype=torch.int8, device=dev)
        self.ppot = torch.empty((batch, blocks, 2, 64), dtype=torch.uint8, device=dev)
        self.out = torch.empty((BH, L, d), dtype=torch.float32, device=dev)

    def scores(self, q, k, stream=None):
        """Quantizes Q and K and fills the P cache."""
        sar_quantize_q(self.p, q, self.qcodes, self.qpot, stream)
        sar_quantize_k(self.p, k, self.kcodes, self.kscale, stream)
        sar_scores(self.p, self.row_ptr, self.cols, self.nnz, self.qcodes, self.qpot, self.kcodes,
                   self.kscale, self.pcodes, self.ppot, stream)

    def apply(self, v, stream=None):
        """Quantizes V and computes O = P_cache V into self.out."""
        sar_quantize_v(self.p, v, self.vcodes_t, self.vscale, stream)
        sar_pv(self.p, self.row_ptr, self.cols, self.nnz, self.pcodes, self.ppot, self.vcodes_t,
               self.vscale, self.out, stream)
        return self.out

    def cached_step(self, q, k, v, stream=None):
        self.scores(q, k, stream)
        return self.apply(v, stream)

    def reused_step(self, v, stream=None):
        return self.apply(v, stream)
