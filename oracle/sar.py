"""CPU oracle for Sparse Attention Reuse with FMDQ-INT8 operands.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (the HIP library and its Python binding) never calls it, and this module
imports nothing from the product path.

Source: "DSTAR: Accelerating Diffusion Transformers via Spatial and Temporal
Redundancy Reduction" (arXiv 2607.15846, HTML version), cited as "DSTAR".

What an attention layer computes under SAR (DSTAR §3.2 "Approach", Fig. 8;
§4.3 "Attention Operation", Fig. 13):

* A static block mask per head (found offline by profiling, §3.2) says which
  (query block, key block) pairs of the score matrix are computed at all.
* Cached step: the block-sparse scores S = Q K^T on the kept blocks, a row
  softmax over the kept keys, the resulting attention matrix P stored in the
  cache, and O = P V.
* Reused steps: Q, K and the softmax are skipped; O = P_cache V_t with the
  current V.
* Every matrix product runs on INT8 operands; the activation operand is
  quantized with FMDQ at a single 8-bit precision (§4.3).

Readings of points the page leaves open (each listed in the design notes):

* Operand roles.  Of each product, the operand whose contraction index runs
  along its sub-channels is the FMDQ "activation" (Q for Q K^T, P for P V); the
  other (K, V) takes the part of the 8-bit weight of the MPU (§4.2 "Design of
  MPU": 2-bit activation slices times 8-bit weights, an inverse quantization
  unit applying one scale per output column): symmetric int8 with one scale per
  output column (per key for K, per head channel for V), scale = max|x| / 127.
* FMDQ-INT8: every sub-channel is 8-bit (PCeil 64, as for the 8-bit
  sub-channels of the linear path), PoT by the same bins against a static base
  (closed upper edges, floor 0, cap 21), step base·2^(PoT−6), codes
  rint(fl32(fl32(x·inv_base)·2^−e)) clipped to ±64.  Sub-channels are one
  token tile of 32 query rows by one channel (Q) or one key (P).
* Mask blocks are 64 × 64 (the 64-wide QPU vectors and PE array of §4.2); a
  query block holds two token tiles.  A query block with no kept key block has
  P = 0 and O = 0.
* Scores are exact integers times scales: S_int = Σ_c (q·2^PoT)·kq, and the
  logit is z = fl32(f64(S_int) · f_s) with f_s = f64(kscale_s) · g and
  g = (f64(base_q)·2^−6)·f64(sm_scale).
* Softmax, written so that both implementations take every integer decision
  (the P codes) from the same bits: x = fl32(z − max_row z); e = exp32(x), a
  float32 exponential by Cody and Waite's range reduction (W. J. Cody, W.
  Waite, "Software Manual for the Elementary Functions", 1980) and a degree-7
  Taylor polynomial by Horner's rule in fused multiply-adds (one rounding to
  float32 per step, IEEE 754 fusedMultiplyAdd), every step in a fixed order;
  E = rint(e·2^36) as an integer (x < −26 gives 0), summed exactly per row;
  P = fl32(f64(E) · (1 / f64(ΣE))).
* Outputs: O = fl32(f64(O_int) · h_c) with O_int = Σ_s (q_P·2^PoT_P)·vq[s][c]
  exact in int64 and h_c = f64(vscale_c) · (f64(base_p)·2^−6).

Layouts (B batch, H heads, L tokens, d head channels, nb = L / 64 blocks):
Q, K, V are float32 [B·H][L][d] (batch-major, then head).  The mask of head h
is kept as compressed rows over (h, query block): row_ptr [H·nb + 1], cols
[nnz] ascending.  The cache holds, for batch b and kept block j, the codes
[64 rows][64 keys] int8 at pcodes[b][j] and the PoT of each (tile, key)
sub-channel at ppot[b][j][2][64].
"""
from __future__ import annotations

import numpy as np

SAR_BLOCK = 64          # mask block edge (queries and keys)
SAR_TILE = 32           # FMDQ token tile of the attention operands
PCEIL8 = 64             # 8-bit precision ceiling (2^(8-2))
P8 = 6                  # log2(PCEIL8)
POT_HI = 21             # PoT cap, as in the linear path
W8_MAX = 127            # symmetric int8 weight-side codes
EXP_FRAC = 36           # fixed-point fraction bits of the exponentials
EXP_X_MIN = np.float32(-26.0)   # exp32(x) below this is 0 (rint(e·2^36) = 0 anyway)

# exp32 constants (float32): log2(e); ln 2 split so that n·LN2_HI is exact.
LOG2E = np.float32(1.4426950408889634)
LN2_HI = np.float32(0.693359375)
LN2_LO = np.float32(0.6931471805599453 - 0.693359375)
EXP_COEF = tuple(np.float32(1.0 / f) for f in (5040.0, 720.0, 120.0, 24.0, 6.0, 2.0, 1.0, 1.0))


# ---------------------------------------------------------------- masks

def mask_to_csr(mask: np.ndarray):
    """Block mask [H][nb][nb] (bool) → (row_ptr int32 [H·nb+1], cols int32 [nnz]).
    Rows are (head, query block) in order; columns ascend within a row."""
    H, nb, nb2 = mask.shape
    assert nb == nb2
    rows = mask.reshape(H * nb, nb)
    counts = rows.sum(axis=1).astype(np.int64)
    row_ptr = np.zeros(H * nb + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(counts)
    cols = np.nonzero(rows)[1].astype(np.int32)   # row-major order: ascending per row
    return row_ptr, cols


# ---------------------------------------------------------------- exp32

def fma32(a, b, c) -> np.ndarray:
    """fl32(a·b + c) with a single rounding (IEEE 754 fusedMultiplyAdd, round to
    nearest, ties to even) for float32 a, b, c of normal magnitude.

    a·b is exact in float64 (24 + 24 significant bits).  s = fl64(a·b + c) and
    its remainder e (Knuth's TwoSum) give a·b + c = s + e exactly.  Rounding s
    to float32 gives the right answer unless s is itself a float32 midpoint and
    e ≠ 0: no other float32 midpoint can lie between s and s + e, since s is
    the float64 nearest to s + e.  At such a midpoint the exact value lies on
    e's side."""
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    b64 = np.asarray(b, dtype=np.float32).astype(np.float64)
    c64 = np.asarray(c, dtype=np.float32).astype(np.float64)
    prod = a64 * b64
    s = prod + c64
    bv = s - prod
    e = (prod - (s - bv)) + (c64 - bv)
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    nb = np.nextafter(r, np.where(s > r64, np.float32(np.inf), np.float32(-np.inf)).astype(np.float32))
    nb64 = nb.astype(np.float64)
    tie = (s != r64) & (s == (r64 + nb64) * 0.5) & (e != 0)
    fixed = np.where(e > 0, np.maximum(r64, nb64), np.minimum(r64, nb64)).astype(np.float32)
    return np.where(tie, fixed, r).astype(np.float32)


def exp32(x: np.ndarray) -> np.ndarray:
    """e^x for float32 x ≤ 0, in float32 with a fixed sequence of roundings:
    n = rint(x·log2 e); r = (x − n·LN2_HI) − n·LN2_LO (Cody–Waite; the first
    difference is exact, the second one fused multiply-add); p(r) the degree-7
    Taylor polynomial of e^r by Horner's rule, one fused multiply-add per
    coefficient; e = p·2^n.  Values below EXP_X_MIN give 0."""
    x = np.asarray(x, dtype=np.float32)
    xs = np.maximum(x, EXP_X_MIN)
    n = np.rint(xs * LOG2E).astype(np.float32)
    r = fma32(-n, LN2_LO, xs - n * LN2_HI)
    p = np.full_like(r, EXP_COEF[0])
    for c in EXP_COEF[1:]:
        p = fma32(p, r, c)
    e = np.ldexp(p, n.astype(np.int32)).astype(np.float32)
    return np.where(x < EXP_X_MIN, np.float32(0.0), e).astype(np.float32)


def exp_fixed(x: np.ndarray) -> np.ndarray:
    """E = rint(exp32(x)·2^EXP_FRAC) as int64 (exact: a power-of-two scaling of
    a float32, then round-half-even to an integer)."""
    e = exp32(x)
    return np.rint(np.ldexp(e, EXP_FRAC).astype(np.float32)).astype(np.int64)


# ---------------------------------------------------------------- quantizers

def pot_int8(m: np.ndarray, base: float) -> np.ndarray:
    """PoT = smallest j in [0, POT_HI] with m ≤ fl32(base·2^j), else POT_HI
    (DSTAR §3.1 Eq. 3, with the linear path's bin edges)."""
    m = np.asarray(m, dtype=np.float32)
    edges = np.ldexp(np.float32(base), np.arange(POT_HI, dtype=np.int32)).astype(np.float32)
    return (m[..., None] > edges).sum(axis=-1).astype(np.int64)


def fmdq_int8_codes(x: np.ndarray, pot: np.ndarray, base: float) -> np.ndarray:
    """q = clip(rint(fl32(fl32(x·inv_base)·2^−e)), ±64), e = PoT − 6, with
    inv_base = fl32(1 / f64(base)) (DSTAR Eq. 2 and Eq. 5 at 8 bits)."""
    inv = np.float32(1.0 / float(np.float32(base)))
    e = np.asarray(pot) - P8
    scale = np.ldexp(np.float32(1.0), (-e).astype(np.int32)).astype(np.float32)
    r = (np.asarray(x, dtype=np.float32) * inv).astype(np.float32) * scale
    return np.clip(np.rint(r.astype(np.float32)), -PCEIL8, PCEIL8).astype(np.int64)


def quantize_q(q: np.ndarray, base_q: float):
    """FMDQ-INT8 of Q [BH][L][d]: per (32-row tile, channel) sub-channel the
    max |Q|, its PoT and the codes.  Returns (codes int64 [BH][L][d], pot int64
    [BH][L/32][d])."""
    BH, L, d = q.shape
    assert L % SAR_TILE == 0
    qt = np.asarray(q, dtype=np.float32).reshape(BH, L // SAR_TILE, SAR_TILE, d)
    m = np.abs(qt).max(axis=2)                         # [BH][tiles][d]
    pot = pot_int8(m, base_q)
    codes = fmdq_int8_codes(qt, pot[:, :, None, :], base_q)
    return codes.reshape(BH, L, d), pot


def weight_scale(amax: np.ndarray) -> np.ndarray:
    """scale = fl32(f64(max|x|) / 127)."""
    return (np.asarray(amax, dtype=np.float64) / W8_MAX).astype(np.float32)


def weight_codes(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """q = clip(rint(f64(x) / f64(scale)), ±127); 0 where the scale is 0."""
    s = np.asarray(scale, dtype=np.float64)
    safe = np.where(s > 0, s, 1.0)
    q = np.clip(np.rint(np.asarray(x, dtype=np.float64) / safe), -W8_MAX, W8_MAX)
    return np.where(s > 0, q, 0.0).astype(np.int64)


def quantize_k(k: np.ndarray):
    """int8 of K [BH][L][d] with one scale per key (the output columns of
    Q K^T).  Returns (codes [BH][L][d], scale float32 [BH][L])."""
    k = np.asarray(k, dtype=np.float32)
    scale = weight_scale(np.abs(k).max(axis=2))
    return weight_codes(k, scale[:, :, None]), scale


def quantize_v(v: np.ndarray):
    """int8 of V [BH][L][d] with one scale per head channel (the output
    columns of P V).  Returns (codes [BH][L][d], scale float32 [BH][d])."""
    v = np.asarray(v, dtype=np.float32)
    scale = weight_scale(np.abs(v).max(axis=1))
    return weight_codes(v, scale[:, None, :]), scale


# ---------------------------------------------------------------- steps

def _blocks_of(row_ptr, cols, h, qb, nb):
    r = h * nb + qb
    return cols[row_ptr[r]:row_ptr[r + 1]]


def scores(qcodes, qpot, kcodes, kscale, row_ptr, cols, heads, base_q, sm_scale, base_p):
    """Cached step, scores to cache (DSTAR §3.2 Fig. 8 cached step; §4.3 Fig.
    13(a)): per kept block the exact S_int, the logits, the row softmax over the
    kept keys, and FMDQ-INT8 of P.  Returns (pcodes int8 [B][nnz][64][64],
    ppot uint8 [B][nnz][2][64], and the float32 P of the kept blocks
    [B][nnz][64][64] for the tests)."""
    BH, L, d = qcodes.shape
    B = BH // heads
    nb = L // SAR_BLOCK
    nnz = len(cols)
    g = (float(np.float32(base_q)) * 2.0 ** -P8) * float(np.float32(sm_scale))
    pcodes = np.zeros((B, nnz, SAR_BLOCK, SAR_BLOCK), dtype=np.int8)
    ppot = np.zeros((B, nnz, 2, SAR_BLOCK), dtype=np.uint8)
    pval = np.zeros((B, nnz, SAR_BLOCK, SAR_BLOCK), dtype=np.float32)
    for bh in range(BH):
        b, h = divmod(bh, heads)
        a_q = qcodes[bh].astype(np.int64) * (np.int64(1) << np.repeat(qpot[bh], SAR_TILE, axis=0))
        f = kscale[bh].astype(np.float64) * g                       # per key
        for qb in range(nb):
            kbs = _blocks_of(row_ptr, cols, h, qb, nb)
            if len(kbs) == 0:
                continue
            j0 = row_ptr[h * nb + qb]
            rows = slice(qb * SAR_BLOCK, (qb + 1) * SAR_BLOCK)
            keys = np.concatenate([np.arange(kb * SAR_BLOCK, (kb + 1) * SAR_BLOCK) for kb in kbs])
            # Exact integer scores (an int64 matmul of integers; every partial
            # sum is below 2^41).
            s_int = a_q[rows] @ kcodes[bh][keys].astype(np.int64).T
            z = (s_int.astype(np.float64) * f[keys][None, :]).astype(np.float32)
            x = (z - z.max(axis=1, keepdims=True)).astype(np.float32)
            E = exp_fixed(x)
            inv = 1.0 / E.sum(axis=1).astype(np.float64)
            P = (E.astype(np.float64) * inv[:, None]).astype(np.float32)
            for i, kb in enumerate(kbs):
                Pb = P[:, i * SAR_BLOCK:(i + 1) * SAR_BLOCK]
                pval[b, j0 + i] = Pb
                for t in range(2):
                    tile = Pb[t * SAR_TILE:(t + 1) * SAR_TILE]
                    pot = pot_int8(tile.max(axis=0), base_p)
                    ppot[b, j0 + i, t] = pot
                    pcodes[b, j0 + i, t * SAR_TILE:(t + 1) * SAR_TILE] = \
                        fmdq_int8_codes(tile, pot[None, :], base_p)
    return pcodes, ppot, pval


def pv(pcodes, ppot, vcodes, vscale, row_ptr, cols, heads, base_p):
    """O = P̂ V̂ over the kept blocks (DSTAR §3.2 cached and reused steps; §4.3
    Fig. 13(b)): O_int exact in int64, then O = fl32(f64(O_int)·h_c).
    Returns float32 [BH][L][d]."""
    BH, L, d = vcodes.shape
    nb = L // SAR_BLOCK
    out = np.zeros((BH, L, d), dtype=np.float32)
    for bh in range(BH):
        b, h = divmod(bh, heads)
        hc = vscale[bh].astype(np.float64) * (float(np.float32(base_p)) * 2.0 ** -P8)
        vq = vcodes[bh].astype(np.int64)
        for qb in range(nb):
            kbs = _blocks_of(row_ptr, cols, h, qb, nb)
            if len(kbs) == 0:
                continue
            j0 = row_ptr[h * nb + qb]
            o_int = np.zeros((SAR_BLOCK, d), dtype=np.int64)
            for i, kb in enumerate(kbs):
                pot = ppot[b, j0 + i].astype(np.int64)                    # [2][64]
                a_p = pcodes[b, j0 + i].astype(np.int64) * (np.int64(1) << np.repeat(pot, SAR_TILE, axis=0))
                o_int += a_p @ vq[kb * SAR_BLOCK:(kb + 1) * SAR_BLOCK]
            out[bh, qb * SAR_BLOCK:(qb + 1) * SAR_BLOCK] = (o_int.astype(np.float64) * hc[None, :]).astype(np.float32)
    return out


def cached_step(q, k, v, row_ptr, cols, heads, base_q, sm_scale, base_p):
    """Cached step: quantize Q, K, V; scores → P cache; O = P̂ V̂."""
    qc, qp = quantize_q(q, base_q)
    kc, ks = quantize_k(k)
    vc, vs = quantize_v(v)
    pc, pp, pval = scores(qc, qp, kc, ks, row_ptr, cols, heads, base_q, sm_scale, base_p)
    o = pv(pc, pp, vc, vs, row_ptr, cols, heads, base_p)
    return dict(qcodes=qc, qpot=qp, kcodes=kc, kscale=ks, vcodes=vc, vscale=vs,
                pcodes=pc, ppot=pp, p=pval, o=o)


def reused_step(pcodes, ppot, v, row_ptr, cols, heads, base_p):
    """Reused step: quantize the current V; O = P_cache V̂_t."""
    vc, vs = quantize_v(v)
    return dict(vcodes=vc, vscale=vs, o=pv(pcodes, ppot, vc, vs, row_ptr, cols, heads, base_p))
