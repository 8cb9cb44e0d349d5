"""Seeded synthetic inputs for the FMDQ differential linear layer.

This module only draws random inputs: activations of two adjacent timesteps,
int8 weights with per-output-channel scales, the cached output of the previous
step and the static base scale.  It holds none of the layer's arithmetic, and
both the HIP path's tests and the CPU oracle take their inputs from here.

The shapes stand in for the linear layers of the diffusion transformers that
DSTAR (arXiv 2607.15846, §5.1 "Algorithm and Workloads") evaluates; its
datasets and trained weights are not used.  Recipe (every draw in float64,
then cast):

* per-input-channel scale c_k = exp(U(ln lo, ln hi));
* X_{t-1} = N(0,1) · c_k; a timestep pair adds Δ = N(0,1) · σ, with
  σ = a · c_k on ordinary sub-channels and σ = 0.5 · c_k on a seeded "heavy"
  set of (token tile × channel) sub-channels; X_t = fl32(X_{t-1} + Δ);
* a multi-pair workload is a random walk: X_p = fl32(X_{p-1} + Δ_p);
* W uniform integers in [-127, 127]; w_scale ~ U[1e-3, 1e-2]; Y_{t-1} ~ N(0,1);
* base = fl32(0.03 · median(c) / 2), the median taken in float64.

Seeds: numpy PCG64 from SeedSequence([0xD57A2607, cfg, layer, pair, stream]).
"""
from __future__ import annotations

import numpy as np

SEED_TAG = 0xD57A2607
S_C, S_X0, S_HEAVY, S_DELTA, S_W, S_WS, S_Y0, S_FRAME = range(8)

#: The five workloads.  rows = batch · tokens, flattened batch-major.
CONFIGS = {
    0: dict(name="dit-xl2-256px", rows=256, tokens_per_seq=256, token_tile=32,
            layers={"fc1": (1152, 4608)}, pairs=1, c_range=(0.5, 8.0),
            heavy=0.03, sigma=0.03, decay=None, text_rows=None, frame=None),
    1: dict(name="pixart-alpha-1024px", rows=8192, tokens_per_seq=4096, token_tile=32,
            layers={"fc1": (1152, 4608), "fc2": (4608, 1152)}, pairs=20,
            c_range=(0.5, 8.0), heavy=0.03, sigma=0.03, decay=25.0,
            text_rows=None, frame=None),
    2: dict(name="sd3-joint-block", rows=4250, tokens_per_seq=4250, token_tile=32,
            layers={"qkv": (1536, 4608), "fc1": (1536, 6144), "fc2": (6144, 1536)},
            pairs=28, c_range=(0.5, 8.0), heavy=0.05, sigma=0.03, decay=None,
            text_rows=(4096, 4250), frame=None),
    3: dict(name="latte-video-16x1024", rows=16384, tokens_per_seq=16384, token_tile=64,
            layers={"fc1": (1152, 4608), "fc2": (4608, 1152)}, pairs=1,
            c_range=(0.5, 8.0), heavy=0.03, sigma=None, decay=None,
            text_rows=None, frame=(1024, 0.01, 0.08)),
    4: dict(name="flux-large", rows=4608, tokens_per_seq=4608, token_tile=32,
            layers={"fc1": (3072, 12288), "fc2": (12288, 3072)}, pairs=28,
            c_range=(0.5, 64.0), heavy=0.08, sigma=0.03, decay=None,
            text_rows=None, frame=None),
}

#: Threshold exponent k0 (Thr_0 = base · 2^k0) used by every workload.
DEFAULT_K0 = 2


def rng(cfg: int, layer: int, pair: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([SEED_TAG, cfg, layer, pair, stream])))


def _heavy_mask(spec: dict, g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    """Boolean [n_tiles][K]: which (token tile × channel) sub-channels are heavy."""
    T = spec["token_tile"]
    nt = (rows + T - 1) // T
    total = int(round(spec["heavy"] * nt * K))
    mask = np.zeros(nt * K, dtype=bool)
    if spec["text_rows"] is not None:
        lo, hi = spec["text_rows"]
        t0, t1 = lo // T, (hi + T - 1) // T
        mask.reshape(nt, K)[t0:t1] = True
        rest = np.flatnonzero(~mask)
        extra = max(0, total - int(mask.sum()))
        mask[g.choice(rest, size=extra, replace=False)] = True
    else:
        mask[g.choice(nt * K, size=total, replace=False)] = True
    return mask.reshape(nt, K)


def _sigma_scale(spec: dict, cfg: int, li: int, pair: int, rows: int) -> np.ndarray:
    """Per-row multiplier a of the ordinary Δ spread (σ = a · c_k)."""
    if spec["frame"] is not None:
        frame_len, lo, hi = spec["frame"]
        nf = (rows + frame_len - 1) // frame_len
        a_f = rng(cfg, li, pair, S_FRAME).uniform(lo, hi, size=nf)
        return np.repeat(a_f, frame_len)[:rows]
    a = spec["sigma"]
    if spec["decay"] is not None:
        a = a * (1.0 - pair / spec["decay"])
    return np.full(rows, a)


def _delta(spec, cfg, li, pair, rows, K, c):
    T = spec["token_tile"]
    heavy = _heavy_mask(spec, rng(cfg, li, pair, S_HEAVY), rows, K)
    a = _sigma_scale(spec, cfg, li, pair, rows)
    heavy_scale = 0.5
    if spec["decay"] is not None:
        heavy_scale = heavy_scale * (1.0 - pair / spec["decay"])
    z = rng(cfg, li, pair, S_DELTA).standard_normal((rows, K))
    sig = a[:, None] * c[None, :]
    hrow = np.repeat(heavy, T, axis=0)[:rows]
    sig = np.where(hrow, heavy_scale * c[None, :], sig)
    return z * sig


def make_inputs(cfg: int, layer: str, pair: int = 1, rows: int | None = None) -> dict:
    """Inputs of one linear layer of workload ``cfg`` at timestep pair ``pair``
    (pair p compares steps p-1 and p of the walk; pairs start at 1).

    ``rows`` truncates the token dimension (the first rows of the full draw are
    kept), for tests that need a slice of a full-size workload.
    """
    spec = CONFIGS[cfg]
    names = list(spec["layers"])
    li = names.index(layer)
    K, N = spec["layers"][layer]
    full_rows = spec["rows"]
    lo, hi = spec["c_range"]
    c = np.exp(rng(cfg, li, 0, S_C).uniform(np.log(lo), np.log(hi), size=K))
    x = (rng(cfg, li, 0, S_X0).standard_normal((full_rows, K)) * c[None, :]).astype(np.float32)
    x_prev = x
    for p in range(1, pair + 1):
        x_prev = x
        x = (x.astype(np.float64) + _delta(spec, cfg, li, p, full_rows, K, c)).astype(np.float32)
    w = rng(cfg, li, 0, S_W).integers(-127, 128, size=(K, N), dtype=np.int64).astype(np.int8)
    w_scale = rng(cfg, li, 0, S_WS).uniform(1e-3, 1e-2, size=N).astype(np.float32)
    y_prev = rng(cfg, li, pair, S_Y0).standard_normal((full_rows, N)).astype(np.float32)
    base = np.float32(0.03 * float(np.median(c)) / 2.0)
    r = full_rows if rows is None else rows
    return dict(x_t=np.ascontiguousarray(x[:r]), x_prev=np.ascontiguousarray(x_prev[:r]),
                w=w, w_scale=w_scale, y_prev=np.ascontiguousarray(y_prev[:r]),
                base=base, k0=DEFAULT_K0, token_tile=spec["token_tile"],
                rows=r, tokens_per_seq=min(spec["tokens_per_seq"], r), K=K, N=N,
                name=f"{spec['name']}/{layer}")


def make_custom(rows: int, K: int, N: int, token_tile: int, seed: int,
                heavy: float = 0.03, c_range=(0.5, 8.0), sigma: float = 0.03,
                k0: int = DEFAULT_K0, tokens_per_seq: int | None = None,
                zero_delta: bool = False) -> dict:
    """Small inputs with the same recipe at any shape (for tests)."""
    spec = dict(token_tile=token_tile, heavy=heavy, text_rows=None, frame=None,
                sigma=sigma, decay=None)
    cfg, li = 1000 + seed, 0
    lo, hi = c_range
    c = np.exp(rng(cfg, li, 0, S_C).uniform(np.log(lo), np.log(hi), size=K))
    x_prev = (rng(cfg, li, 0, S_X0).standard_normal((rows, K)) * c[None, :]).astype(np.float32)
    if zero_delta:
        x_t = x_prev.copy()
    else:
        x_t = (x_prev.astype(np.float64) + _delta(spec, cfg, li, 1, rows, K, c)).astype(np.float32)
    w = rng(cfg, li, 0, S_W).integers(-127, 128, size=(K, N), dtype=np.int64).astype(np.int8)
    w_scale = rng(cfg, li, 0, S_WS).uniform(1e-3, 1e-2, size=N).astype(np.float32)
    y_prev = rng(cfg, li, 1, S_Y0).standard_normal((rows, N)).astype(np.float32)
    base = np.float32(0.03 * float(np.median(c)) / 2.0)
    return dict(x_t=x_t, x_prev=x_prev, w=w, w_scale=w_scale, y_prev=y_prev,
                base=base, k0=k0, token_tile=token_tile, rows=rows,
                tokens_per_seq=rows if tokens_per_seq is None else tokens_per_seq,
                K=K, N=N, name=f"custom-{rows}x{K}x{N}-T{token_tile}-s{seed}")


def make_walk(cfg: int, layer: str, pairs: int) -> list:
    """X_0, X_1, ..., X_pairs of the random walk of one layer of workload
    ``cfg``, drawn once (make_inputs(cfg, layer, p) has X_{p-1} and X_p)."""
    spec = CONFIGS[cfg]
    names = list(spec["layers"])
    li = names.index(layer)
    K, _ = spec["layers"][layer]
    full_rows = spec["rows"]
    lo, hi = spec["c_range"]
    c = np.exp(rng(cfg, li, 0, S_C).uniform(np.log(lo), np.log(hi), size=K))
    x = (rng(cfg, li, 0, S_X0).standard_normal((full_rows, K)) * c[None, :]).astype(np.float32)
    xs = [x]
    for p in range(1, pairs + 1):
        x = (x.astype(np.float64) + _delta(spec, cfg, li, p, full_rows, K, c)).astype(np.float32)
        xs.append(x)
    return xs


def profiled_base(delta: np.ndarray) -> np.float32:
    """A static base "profiled" from one observed difference, by the same rule
    as the workloads' own base: half the median over channels of the
    per-channel RMS of Δ (the workloads draw Δ with RMS σ = 0.03·c_k and use
    0.03·median(c)/2).  For layers whose input is produced by another layer
    (the second linear of an MLP), where no c_k is drawn."""
    d = np.asarray(delta, dtype=np.float64)
    rms = np.sqrt(np.mean(d * d, axis=0))
    return np.float32(float(np.median(rms)) / 2.0)
