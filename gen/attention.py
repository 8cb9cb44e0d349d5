"""Seeded synthetic inputs for Sparse Attention Reuse (SAR) attention layers.

This module only draws random inputs: Q, K, V of one attention layer at two
adjacent timesteps, a static block mask per head and the layer's static
scales.  It holds none of the attention arithmetic; the HIP path's tests and
the CPU oracle both take their inputs from here.

The workload stands in for the self-attention of PixArt-α at 1024 px (two
images of 4096 tokens, 16 heads of 72 channels), the model family DSTAR
(arXiv 2607.15846) profiles in §3.2 (Fig. 7) and evaluates in §5; its prompts,
seeds and trained weights are not used.  Recipe (every draw in float64, then
cast to float32):

* per (head, channel) scale c = exp(U(ln 0.5, ln 2)), shared by Q and K;
* Q = N(0,1)·c, K = N(0,1)·c, V = N(0,1) per element; the next timestep's
  V_t = V + N(0,1)·0.05 (adjacent steps are similar, §2.2);
* block mask per head (64 × 64 blocks): the diagonal band |qb − kb| ≤ 1 and
  the first key block are always kept, the remaining blocks are kept with the
  probability that brings the kept fraction to `density` (DSTAR Table 1: 37%
  of the blocks pruned, i.e. density 0.63);
* base_q = fl32(median over (head, channel) of max |Q| / 64), the static base
  profiled from the data (the median in float64); base_p = 2^-15 (softmax
  outputs are at most 1); sm_scale = fl32(1/sqrt(d)).

Seeds: numpy PCG64 from SeedSequence([0xD57A2608, seed, stream]).
"""
from __future__ import annotations

import numpy as np

SEED_TAG = 0xD57A2608
S_C, S_Q, S_K, S_V, S_DV, S_MASK = range(6)
BLOCK = 64

#: Attention workloads: batch, heads, tokens per image, head channels, density.
ATTN_CONFIGS = {
    "pixart-alpha-1024px-attn": dict(batch=2, heads=16, L=4096, d=72, density=0.63),
    "small": dict(batch=1, heads=2, L=256, d=72, density=0.63),
}


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_TAG, seed, stream])))


def make_mask(heads: int, L: int, density: float, seed: int) -> np.ndarray:
    """Block mask [heads][nb][nb] (bool) with the structure described above."""
    nb = L // BLOCK
    g = rng(seed, S_MASK)
    qb = np.arange(nb)[:, None]
    kb = np.arange(nb)[None, :]
    fixed = (np.abs(qb - kb) <= 1) | (kb == 0)
    frac_fixed = fixed.mean()
    p = 0.0 if density <= frac_fixed else min(1.0, (density - frac_fixed) / (1.0 - frac_fixed))
    mask = np.empty((heads, nb, nb), dtype=bool)
    for h in range(heads):
        mask[h] = fixed | (g.random((nb, nb)) < p)
    return mask


def make_attention(batch: int, heads: int, L: int, d: int, density: float, seed: int) -> dict:
    """Q, K, V, V_next float32 [batch·heads][L][d], mask, base_q, base_p, sm_scale."""
    assert L % BLOCK == 0
    BH = batch * heads
    c = np.exp(rng(seed, S_C).uniform(np.log(0.5), np.log(2.0), size=(heads, d)))
    cb = np.tile(c, (batch, 1))[:, None, :]                      # [BH][1][d]
    q = (rng(seed, S_Q).standard_normal((BH, L, d)) * cb).astype(np.float32)
    k = (rng(seed, S_K).standard_normal((BH, L, d)) * cb).astype(np.float32)
    v = rng(seed, S_V).standard_normal((BH, L, d))
    v_next = (v + rng(seed, S_DV).standard_normal((BH, L, d)) * 0.05).astype(np.float32)
    v = v.astype(np.float32)
    amax = np.abs(q.astype(np.float64)).max(axis=1)               # [BH][d]
    base_q = np.float32(np.median(amax) / 64.0)
    return dict(batch=batch, heads=heads, L=L, d=d, q=q, k=k, v=v, v_next=v_next,
                mask=make_mask(heads, L, density, seed), base_q=base_q,
                base_p=np.float32(2.0 ** -15), sm_scale=np.float32(1.0 / np.sqrt(d)))


def make_config(name: str, seed: int = 1) -> dict:
    s = ATTN_CONFIGS[name]
    return make_attention(s["batch"], s["heads"], s["L"], s["d"], s["density"], seed)
