"""CPU oracle for the FMDQ differential linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (the HIP library and its Python binding) never calls it, and this module
imports nothing from the product path.

Source: "DSTAR: Accelerating Diffusion Transformers via Spatial and Temporal
Redundancy Reduction" (arXiv 2607.15846, HTML version), cited below as
"DSTAR".  Section, equation and figure numbers refer to that page.

What the layer computes (DSTAR §2.2 Eq. 1; §3.1 steps ❶ ❸ ❹ ❺; §4.2 "Design of
MPU", "Design of QPU"; §4.3 "Linear Operation"):

    Δ        = X_t − X_{t−1}                                    (Eq. 1)
    M_{τk}   = max |Δ| over the rows of token tile τ, channel k  (§3.1 ❶)
    PoT_{τk} = ⌈log2(M_{τk} / base)⌉  (Eq. 3), floored at 0, capped at POT_HI
    bits     = 2/4/6/8 by binning M against Thr_0·4^N            (§3.1 ❶)
    q        = round(Δ · s),  s = PCeil / (base · 2^PoT)         (Eq. 2)
    groups   = sub-channels of a tile sorted by FPoT (Eq. 4)     (§3.1 ❸)
    acc_g    = Σ_{k in group g} q · W                            (§3.1 ❺)
    S        = partial sums of the groups aligned by left shifts (§3.1 ❷/❺, Fig. 6)
    Y_t      = Y_{t−1} + w_scale · base · S                      (§4.2 inverse
               quantization unit; §4.3 reverse differential fused into the GEMM)

Readings of points the page leaves open (each is listed, with its reason, in
the design notes of this repository):

* PCeil of a b-bit sub-channel is 2^(b−2): 1, 4, 16, 64.  It gives PCeil = 1 for
  2 bits as in the worked example of §3.1 ❶, ranges exactly 4× apart as the
  thresholds Thr_0·2^(2N) of §3.1 ❶ say, and integer FPoT, which is what lets
  partial sums be aligned by shifts alone.
* Thr_0 = base · 2^k0 with an integer k0 ("thr0_log2"); precision then follows
  from PoT alone, which is the bin-plus-lookup-table of §4.2 QPU stage 2.
* PoT = the smallest j in [0, POT_HI] with M ≤ base·2^j (closed upper bin edge,
  as the worked example's interval [0, 2^0]); POT_HI when none qualifies.
* Instead of FPoT (which is not an integer when base is not a power of two),
  every sub-channel carries the integer tag  tag = (b−2) − PoT + 15  in [0, 15].
  tag − FPoT is the same constant for every sub-channel of a layer, so ascending
  tag is ascending FPoT and tag differences are FPoT differences.  The step of
  a sub-channel is δ = base · 2^e with e = 15 − tag = PoT − (b−2).
* Codes: r = fl32(fl32(Δ · inv_base) · 2^−e) with inv_base = fl32(1/base) formed
  once in float64; q = round-half-to-even(r) clipped to ±PCeil.  All of it is
  done in float32, the precision of the inputs, so that both implementations
  take the same integer decisions.
* The bucket order: tag ascending (ascending FPoT); inside one FPoT group,
  precision descending, then channel ascending.  DSTAR leaves the order of
  equal FPoTs free (a bitonic network, §3.1 ❸; the Fig. 11 meta table has
  ties that are not index-ordered).  Putting the wider codes of a group first
  makes the sub-channels whose shift-aligned codes exceed 8 bits a prefix of
  every group.
* The per-group sums are exact integers; S = Σ_g acc_g · 2^(15−g) in int64; the
  output is fl32(f64(Y_{t−1}) + (f64(S) · f64(base)) · f64(w_scale[n])).

Parity of every function here is pinned by tests against values printed in
DSTAR, closed forms, library routines and brute force (``tests/test_oracle_*``).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64

#: PCeil per precision (reading of DSTAR §3.1 ❶, Eq. 2): 2^(b-2).
PCEIL = {2: 1, 4: 4, 6: 16, 8: 64}
#: Largest PoT exponent; with it every tag fits in 4 bits.
POT_HI = 21
#: Tag offset: tag = (b - 2) - PoT + TAG_OFF.
TAG_OFF = 15
#: Number of distinct tags (FPoT groups) per token tile.
N_TAGS = 16
#: Precision code stored in bits 4-5 of a tag byte: b / 2 - 1.
PREC_SHIFT = 4
#: Bins of the bucket order: (tag, precision) pairs, four precisions per tag.
N_BINS = 4 * N_TAGS


# --------------------------------------------------------------------------- #
# Step ❶ of DSTAR §3.1 (and Eq. 1): differential, sub-channels, PoT, precision #
# --------------------------------------------------------------------------- #
def differential(x_t: np.ndarray, x_prev: np.ndarray) -> np.ndarray:
    """Δ = X_t − X_{t−1} in float32 (DSTAR §2.2 Eq. 1; §3.1 computation flow)."""
    return np.subtract(x_t.astype(F32), x_prev.astype(F32), dtype=F32)


def n_tiles(rows: int, token_tile: int) -> int:
    """Number of token tiles; the last one may be ragged (DSTAR §3.1 ❶)."""
    return (rows + token_tile - 1) // token_tile


def tile_rows(tile: int, rows: int, token_tile: int) -> tuple[int, int]:
    """[first, last) rows of a token tile; the ragged last tile keeps only real rows."""
    r0 = tile * token_tile
    return r0, min(r0 + token_tile, rows)


def subchannel_max(delta: np.ndarray, token_tile: int) -> np.ndarray:
    """M_{τk}: the largest |Δ| of each sub-channel (tile τ × channel k).

    DSTAR §3.1 ❶ (the largest magnitude within a sub-channel) and §4.2 QPU
    stage 1.  A running maximum over the rows of the tile, in float32.
    """
    rows, K = delta.shape
    nt = n_tiles(rows, token_tile)
    out = np.zeros((nt, K), dtype=F32)
    for tau in range(nt):
        r0, r1 = tile_rows(tau, rows, token_tile)
        m = np.zeros(K, dtype=F32)
        for r in range(r0, r1):
            m = np.maximum(m, np.abs(delta[r]))
        out[tau] = m
    return out


def pot_exponent(m: np.ndarray, base: float) -> np.ndarray:
    """PoT = ⌈log2(M / base)⌉ (DSTAR Eq. 3), floored at 0 and capped at POT_HI.

    Evaluated as the bin operation of DSTAR §4.2 QPU stage 2: the smallest j
    with M ≤ base·2^j, each threshold an exact float32 power-of-two multiple of
    base.  Sub-channels above base·2^POT_HI get POT_HI (their codes clip).
    """
    m = np.asarray(m, dtype=F32)
    base32 = F32(base)
    pot = np.full(m.shape, POT_HI, dtype=np.int32)
    for j in range(POT_HI, -1, -1):
        thr = np.ldexp(base32, j).astype(F32)
        pot = np.where(m <= thr, j, pot)
    return pot


def precision_bits(pot: np.ndarray, k0: int) -> np.ndarray:
    """Bit width from the thresholds Thr_N = Thr_0 · 2^(2N) (DSTAR §3.1 ❶).

    With Thr_0 = base · 2^k0: 2 bits when M ≤ Thr_0, 4 when M ≤ 4·Thr_0, 6 when
    M ≤ 16·Thr_0, else 8.  Because PoT is the smallest j with M ≤ base·2^j,
    "M ≤ base·2^(k0+2N)" is the same test as "PoT ≤ k0 + 2N".
    """
    pot = np.asarray(pot)
    bits = np.full(pot.shape, 8, dtype=np.int32)
    bits = np.where(pot <= k0 + 4, 6, bits)
    bits = np.where(pot <= k0 + 2, 4, bits)
    bits = np.where(pot <= k0, 2, bits)
    return bits


def fpot_tag(bits: np.ndarray, pot: np.ndarray) -> np.ndarray:
    """Integer FPoT tag of a sub-channel: (b − 2) − PoT + 15.

    DSTAR Eq. 4 gives FPoT = log2(PCeil) − PoT − 2·log2(base); with
    PCeil = 2^(b−2) the tag is FPoT + 2·log2(base) + 15, an integer in [0, 15].
    """
    return (np.asarray(bits) - 2) - np.asarray(pot) + TAG_OFF


def step_exponent(tag: np.ndarray) -> np.ndarray:
    """e = 15 − tag: the step of a sub-channel is base·2^e = 1/s (Eq. 2, Eq. 5)."""
    return TAG_OFF - np.asarray(tag)


def inv_base_f32(base: float) -> np.float32:
    """fl32(1 / base), formed once in float64."""
    return F32(1.0 / F64(F32(base)))


def quantize_values(delta: np.ndarray, e: np.ndarray, bits: np.ndarray,
                    inv_base: np.float32) -> np.ndarray:
    """Codes q = clip(round(Δ · s), ±PCeil) with s = 2^−e / base (DSTAR Eq. 2, §3.1 ❶).

    Two float32 products — Δ·inv_base, then an exact scaling by 2^−e — then
    round half to even, then the clip of DSTAR §4.2 QPU stage 3.
    """
    r = np.multiply(delta.astype(F32), inv_base, dtype=F32)
    r = np.multiply(r, np.ldexp(F32(1.0), -np.asarray(e)).astype(F32), dtype=F32)
    q = np.rint(r)
    pceil = np.left_shift(1, np.asarray(bits) - 2).astype(F32)
    q = np.clip(q, -pceil, pceil)
    return q.astype(np.int8)


def quantize(x_t: np.ndarray, x_prev: np.ndarray, token_tile: int, base: float,
             k0: int):
    """Steps ❶ of DSTAR §3.1 for a whole layer input.

    Returns
      codes  int8  [n_t][K][T]   code of row τ·T+t, channel k at [τ][k][t];
                                 rows past the end of a ragged tile are 0
      tags   uint8 [n_t][K]      bits 0-3 tag, bits 4-5 precision code b/2−1
      hist   int64 [4]           number of sub-channels at 2/4/6/8 bits
    """
    rows, K = x_t.shape
    T = token_tile
    delta = differential(x_t, x_prev)
    m = subchannel_max(delta, T)
    pot = pot_exponent(m, base)
    bits = precision_bits(pot, k0)
    tag = fpot_tag(bits, pot)
    e = step_exponent(tag)
    inv_base = inv_base_f32(base)
    nt = m.shape[0]
    codes = np.zeros((nt, K, T), dtype=np.int8)
    for tau in range(nt):
        r0, r1 = tile_rows(tau, rows, T)
        q = quantize_values(delta[r0:r1], e[tau][None, :], bits[tau][None, :], inv_base)
        codes[tau, :, : r1 - r0] = q.T
    tags = (tag | (((bits // 2) - 1) << PREC_SHIFT)).astype(np.uint8)
    hist = np.array([(bits == b).sum() for b in (2, 4, 6, 8)], dtype=np.int64)
    return codes, tags, hist


def tag_of(tags: np.ndarray) -> np.ndarray:
    """Tag (FPoT group) from a tag byte."""
    return (np.asarray(tags) & 0x0F).astype(np.int64)


def bits_of(tags: np.ndarray) -> np.ndarray:
    """Precision in bits from a tag byte."""
    return ((np.asarray(tags).astype(np.int64) >> PREC_SHIFT) & 0x3) * 2 + 2


# --------------------------------------------------------------------------- #
# Step ❸ of DSTAR §3.1: reorder sub-channels of a tile by FPoT                  #
# --------------------------------------------------------------------------- #
def bucket_key(tags: np.ndarray) -> np.ndarray:
    """Sort key of a sub-channel: 4 · tag + (3 − precision code).

    Ascending key = ascending FPoT tag (DSTAR §3.1 ❸), and inside one tag
    descending precision (a free choice: the pages fix only the FPoT order).
    """
    t = np.asarray(tags).astype(np.int64)
    return 4 * (t & 0x0F) + (3 - ((t >> PREC_SHIFT) & 0x3))


def group_bounds(off_tile: np.ndarray, g: int) -> tuple[int, int]:
    """[first, last) positions of FPoT group g in a tile's bucket order."""
    return int(off_tile[4 * g]), int(off_tile[4 * g + 4])


def bucket(tags: np.ndarray):
    """Group the channels of every token tile by tag, in ascending FPoT.

    DSTAR §3.1 ❸ (sub-channels sharing an FPoT placed next to each other, in
    ascending FPoT) and §4.2 QPU stage 4.  Written as a counting sort over the
    64 (tag, precision) bins of ``bucket_key``: count the channels of each bin,
    take the exclusive prefix sum, then place the channels in index order —
    which keeps channel order inside a bin.

    Returns perm uint16 [n_t][K] and group_off int32 [n_t][65]:
    group_off[τ][β] = number of channels of tile τ with key < β.  The channels
    of FPoT group g are perm[τ][group_off[τ][4g] : group_off[τ][4g + 4]],
    widest precision first.
    """
    tags = np.asarray(tags)
    nt, K = tags.shape
    perm = np.zeros((nt, K), dtype=np.uint16)
    off = np.zeros((nt, N_BINS + 1), dtype=np.int32)
    for tau in range(nt):
        key = bucket_key(tags[tau])
        count = np.zeros(N_BINS, dtype=np.int64)
        for k in range(K):
            count[key[k]] += 1
        start = np.zeros(N_BINS + 1, dtype=np.int64)
        for b in range(N_BINS):
            start[b + 1] = start[b] + count[b]
        off[tau] = start
        cursor = start[:N_BINS].copy()
        for k in range(K):
            b = key[k]
            perm[tau, cursor[b]] = k
            cursor[b] += 1
    return perm, off


# --------------------------------------------------------------------------- #
# Step ❺ of DSTAR §3.1 and the MPU of §4.2: grouped GEMM, shifts, dequant      #
# --------------------------------------------------------------------------- #
def group_accumulators(codes_tile: np.ndarray, perm_tile: np.ndarray,
                       off_tile: np.ndarray, w: np.ndarray) -> np.ndarray:
    """acc[g][t][n] = Σ over channels k of group g of q[t][k] · W[k][n].

    One integer accumulator per FPoT group (DSTAR §3.1 ❺; §4.2 "Design of
    MPU").  Each group product is a float64 matmul; every partial sum is an
    integer below 2^53, so the result is exact.  codes_tile is [K][T].
    """
    K, T = codes_tile.shape
    N = w.shape[1]
    acc = np.zeros((N_TAGS, T, N), dtype=np.int64)
    for g in range(N_TAGS):
        lo, hi = group_bounds(off_tile, g)
        if hi == lo:
            continue
        ch = perm_tile[lo:hi].astype(np.int64)
        a = codes_tile[ch, :].T.astype(F64)      # [T][n_g]
        b = w[ch, :].astype(F64)                 # [n_g][N]
        acc[g] = np.rint(a @ b).astype(np.int64)
    return acc


def shift_combine(acc: np.ndarray) -> np.ndarray:
    """S = Σ_g acc_g · 2^(15−g): partial sums aligned by left shifts.

    DSTAR §3.1 ❷/❺ and Fig. 6: partial sums are accumulated in ascending FPoT,
    each shifted left by the FPoT difference to the next group; written out,
    that is the sum of every group shifted to the units of the smallest step
    (tag 15, e = 0).  Exact in int64.
    """
    acc = np.asarray(acc, dtype=np.int64)
    s = np.zeros(acc.shape[1:], dtype=np.int64)
    for g in range(N_TAGS):
        s = s + np.left_shift(acc[g], TAG_OFF - g)
    return s


def dequant_add(s: np.ndarray, base: float, w_scale: np.ndarray,
                y_prev: np.ndarray) -> np.ndarray:
    """Y_t = Y_{t−1} + w_scale · base · S (DSTAR §4.2 inverse quantization and
    accumulation units; §4.3 reverse differential fused into the GEMM).

    f64(S)·f64(base), then ·f64(w_scale[n]), then + f64(Y_{t−1}), rounded once
    to float32.
    """
    d = (np.asarray(s).astype(F64) * F64(F32(base))) * np.asarray(w_scale, dtype=F32).astype(F64)[None, :]
    return (np.asarray(y_prev, dtype=F32).astype(F64) + d).astype(F32)


def linear(codes: np.ndarray, tags: np.ndarray, perm: np.ndarray,
           group_off: np.ndarray, w: np.ndarray, w_scale: np.ndarray,
           y_prev: np.ndarray, base: float, token_tile: int,
           tiles=None, return_acc: bool = False):
    """Differential linear of DSTAR §3.1 ❺ / §4.3 for the token tiles ``tiles``
    (all by default).  Returns Y_t rows of those tiles (float32 [rows][N]) and,
    if asked, the group accumulators {tile: int64 [16][T][N]}.
    """
    rows = y_prev.shape[0]
    T = token_tile
    nt = n_tiles(rows, T)
    if tiles is None:
        tiles = range(nt)
    y = np.array(y_prev, dtype=F32, copy=True)
    accs = {}
    for tau in tiles:
        r0, r1 = tile_rows(tau, rows, T)
        acc = group_accumulators(codes[tau], perm[tau], group_off[tau], w)
        s = shift_combine(acc)
        y[r0:r1] = dequant_add(s[: r1 - r0], base, w_scale, y_prev[r0:r1])
        if return_acc:
            accs[tau] = acc
    if return_acc:
        return y, accs
    return y


#: 2-bit slices (DSTAR §3.1 ❷): slice n of a code sits at FPoT − 2n, i.e.
#: slice tag tag − 2n in [−6, 15]; bin = slice tag + SLICE_TAG_OFF.
SLICE_TAG_OFF = 6
SLICE_BINS = 22


def code_slices(q: np.ndarray, bits: np.ndarray):
    """The 2-bit slices of b-bit codes (DSTAR §3.1 ❷: a code is the sum of its
    slices shifted by 2n), least significant first, b/2 of them.

    Reading for signed codes (the page's example is unsigned): the radix-4
    digits of the two's-complement code — slices below the top one in 0..3,
    the top slice in −2..1 — so q = Σ_n slice_n · 4^n exactly and every slice
    is the 2-bit field (q >> 2n) & 3 (the top one read as signed).
    Returns a list of b_max/2 int64 arrays (zero above a code's own count).
    """
    q = np.asarray(q, dtype=np.int64)
    nsl = np.asarray(bits, dtype=np.int64) // 2
    out = []
    for n in range(4):
        field = (q >> (2 * n)) & 3
        top = (n == nsl - 1)
        val = np.where(top & (field >= 2), field - 4, field)
        out.append(np.where(n < nsl, val, 0))
    return out


def slice_encode(codes: np.ndarray, tags: np.ndarray):
    """Steps ❷ ❸ ❹ of DSTAR §3.1 as a stream per token tile.

    Every b-bit sub-channel becomes b/2 entries (channel k, slice n), the
    slice at slice tag tag − 2n (its FPoT lowered by 2n).  The entries of a
    tile are ordered by slice tag ascending (ascending FPoT), ties by channel
    ascending, and each carries the number of left shifts to apply to the
    running partial sum before it — the slice-tag difference to the previous
    entry (0 for the first), the encoding of ❹.  Returns
      ent   uint32 [n_t][4K]   k | n << 16 | shift << 24 (entries past the
                               tile's count are 0xFFFFFFFF)
      data  uint8  [n_t][4K][T/4]  the slice's 2-bit fields of rows t, four
                               rows per byte (row t at bits 2·(t mod 4))
      off   int32  [n_t][23]   off[τ][β] = entries of tile τ with bin < β
    """
    codes = np.asarray(codes)
    nt, K, T = codes.shape
    tag = tag_of(tags)
    bits = bits_of(tags)
    ent = np.full((nt, 4 * K), 0xFFFFFFFF, dtype=np.uint32)
    data = np.zeros((nt, 4 * K, T // 4), dtype=np.uint8)
    off = np.zeros((nt, SLICE_BINS + 1), dtype=np.int32)
    for tau in range(nt):
        items = []                     # (bin, k, n)
        for k in range(K):
            for n in range(int(bits[tau, k]) // 2):
                items.append((int(tag[tau, k]) - 2 * n + SLICE_TAG_OFF, k, n))
        items.sort()
        slices = code_slices(codes[tau].astype(np.int64), bits[tau][:, None])
        prev = None
        for j, (b, k, n) in enumerate(items):
            shift = 0 if prev is None else b - prev
            prev = b
            ent[tau, j] = k | (n << 16) | (shift << 24)
            field = slices[n][k] & 3                      # the 2-bit pattern
            packed = field.reshape(T // 4, 4) << (2 * np.arange(4))
            data[tau, j] = packed.sum(axis=1).astype(np.uint8)
        for beta in range(SLICE_BINS + 1):
            off[tau, beta] = sum(1 for it in items if it[0] < beta)
    return ent, data, off


#: Constants of the tanh form of GELU: sqrt(2/pi) and the cubic coefficient.
GELU_C = 0.7978845608028654
GELU_A = 0.044715


def gelu(y: np.ndarray) -> np.ndarray:
    """GELU of the MLP between the two linears, the activation DSTAR fuses
    into the linear through its vector unit (§4.2 "Design of VPU", §4.3
    "Linear Operation").  The page gives no formula (its unit uses piecewise
    cubics); the reading here is the tanh form used by the DiT MLPs,
    0.5·y·(1 + tanh(u)) with u = c·(y + a·y³), written as y / (1 + exp(−2u))
    (the same function without the cancellation of 1 + tanh(u) at negative
    y) and evaluated in float64, then rounded once to float32.  The cube is
    (y·y)·y.
    """
    y64 = np.asarray(y, dtype=F32).astype(F64)
    u = GELU_C * (y64 + GELU_A * ((y64 * y64) * y64))
    with np.errstate(over="ignore"):
        return (y64 / (1.0 + np.exp(-2.0 * u))).astype(F32)


def mlp_step(x_t, x_prev, y1_prev, g_prev, y2_prev, fc1, fc2, token_tile, k0):
    """One timestep pair through fc1 → GELU → fc2 with every output cached:
    fc1 updates its output Y1 differentially (layer); G = GELU(Y1) is fc2's
    input at this step and G_prev its input at the previous one, so fc2
    updates Y2 from the difference G − G_prev (DSTAR §2.2 Eq. 1 applied to
    both linears of the MLP; §4.3 fuses the GELU into the first).
    ``fc1``/``fc2`` are dicts with w, w_scale and base.  Returns (y1, g, y2,
    hist1, hist2)."""
    r1 = layer(x_t, x_prev, fc1["w"], fc1["w_scale"], y1_prev, fc1["base"], token_tile, k0)
    g = gelu(r1["y"])
    r2 = layer(g, g_prev, fc2["w"], fc2["w_scale"], y2_prev, fc2["base"], token_tile, k0)
    return r1["y"], g, r2["y"], r1["hist"], r2["hist"]


#: The range a layer's base is held to: the library rejects a static base
#: outside it, and a dynamic base is clamped into it.
BASE_MIN = 2.0 ** -100
BASE_MAX = 2.0 ** 100


def dynamic_base(x_t: np.ndarray, x_prev: np.ndarray, token_tile: int, fallback: float) -> np.float32:
    """The base as DSTAR §3.1 ❶ defines it before the static-base shortcut:
    the smallest sub-channel maximum M_{τk} of the layer input, found in a
    first pass over X (the "DS-FMDQ-DYN" variant of DSTAR §5.2, Table 2).

    Readings of what the page leaves open: sub-channels whose Δ is zero in
    every row are left out (their codes are 0 whatever the base, and a zero
    base has no Eq. 2 scale); if every sub-channel is zero the static base
    ``fallback`` is kept; the minimum is clamped to [BASE_MIN, BASE_MAX].  The
    minimum of float32 values is exact, so both implementations agree bit for
    bit.
    """
    m = subchannel_max(differential(x_t, x_prev), token_tile)
    pos = m[m > 0]
    if pos.size == 0:
        return F32(fallback)
    return F32(min(max(F64(pos.min()), BASE_MIN), BASE_MAX))


def layer_dynamic(x_t, x_prev, w, w_scale, y_prev, fallback_base, token_tile, k0):
    """The layer with the dynamic base: pass 1 finds the base (dynamic_base),
    pass 2 is the static pipeline run with it.  The result carries "base"."""
    base = dynamic_base(x_t, x_prev, token_tile, fallback_base)
    out = layer(x_t, x_prev, w, w_scale, y_prev, base, token_tile, k0)
    out["base"] = base
    return out


def layer(x_t, x_prev, w, w_scale, y_prev, base, token_tile, k0):
    """The whole FMDQ differential linear: quantize, bucket, grouped GEMM."""
    codes, tags, hist = quantize(x_t, x_prev, token_tile, base, k0)
    perm, off = bucket(tags)
    y = linear(codes, tags, perm, off, w, w_scale, y_prev, base, token_tile)
    return dict(codes=codes, tags=tags, hist=hist, perm=perm, group_off=off, y=y)
