"""Pins of the SAR / FMDQ-INT8 attention oracle.

Each test checks the oracle against something other than itself: math.exp
(the float32 exponential), the defining inequalities of the PoT bins and of
rounding (quantizers), closed forms (uniform attention: Q = 0 gives P = 1/n and
O = the mean of the quantized V; one-hot attention through orthogonal
Hadamard keys gives O = the quantized V row of the chosen key), an invariance
(pruned blocks do not matter), pure-Python brute force on tiny shapes (exact
integer scores, float64 softmax, float64 products) and plain float64 masked
attention within the quantization error.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from gen import attention as ga
from oracle import sar


# ---------------------------------------------------------------- exp32

def _f32_nearest(q: Fraction) -> np.float32:
    """The float32 nearest to the rational q, ties to even (brute force over
    the neighbours of a float64 approximation)."""
    f = np.float32(float(q))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    best = min(abs(Fraction(float(c)) - q) for c in cands)
    ties = [c for c in cands if abs(Fraction(float(c)) - q) == best]
    if len(ties) == 1:
        return ties[0]
    return [c for c in ties if (int(np.array(c, np.float32).view(np.uint32)) & 1) == 0][0]


def test_fma32_is_one_rounding_of_the_exact_value():
    rng = np.random.default_rng(7)
    n = 3000
    a = (rng.uniform(-2, 2, n) * 2.0 ** rng.integers(-20, 2, n)).astype(np.float32)
    b = (rng.uniform(-1, 1, n) * 2.0 ** rng.integers(-12, 1, n)).astype(np.float32)
    c = (rng.uniform(-1, 1, n) * 2.0 ** rng.integers(-14, 1, n)).astype(np.float32)
    # exact sums on a float32 midpoint after float64 rounding, where rounding
    # twice (to float64, then to float32) picks the wrong neighbour:
    # (2^-12(1+2^-23))·(2^-12(1-2^-23)) = 2^-24 - 2^-70, and c = 1 + 2^-23 puts
    # a·b + c just below the midpoint 1 + 3·2^-24
    x, y = np.float32(2.0 ** -12 * (1 + 2.0 ** -23)), np.float32(2.0 ** -12 * (1 - 2.0 ** -23))
    a = np.concatenate([a, [x, -x, x, y]]).astype(np.float32)
    b = np.concatenate([b, [y, y, x, y]]).astype(np.float32)
    c = np.concatenate([c, [np.float32(1 + 2.0 ** -23), np.float32(-(1 + 2.0 ** -23)), np.float32(1.0),
                            np.float32(1 + 2.0 ** -23)]]).astype(np.float32)
    got = sar.fma32(a, b, c)
    for i in range(len(a)):
        want = _f32_nearest(Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i])))
        assert got[i] == want, (i, a[i], b[i], c[i], got[i], want)
    # the constructed case differs from two roundings
    two = np.float32(np.float64(x) * np.float64(y) + np.float64(np.float32(1 + 2.0 ** -23)))
    assert got[n] != two and got[n] == np.float32(1 + 2.0 ** -23)


def test_exp32_against_math_exp():
    x = np.concatenate([np.linspace(-26, 0, 200001), -np.logspace(-8, 0, 2000),
                        [0.0, -1e-30, -0.34657359, -0.34657360, -25.999]]).astype(np.float32)
    got = sar.exp32(x).astype(np.float64)
    ref = np.array([math.exp(float(t)) for t in x])
    rel = np.abs(got - ref) / ref
    assert rel.max() <= 4 * 2.0 ** -24, rel.max()
    assert sar.exp32(np.float32(0.0)) == np.float32(1.0)


def test_exp32_cutoff_and_fixed_point():
    x = np.array([-26.0001, -30.0, -87.0, -np.inf], dtype=np.float32)
    assert (sar.exp32(x) == 0).all()
    assert (sar.exp_fixed(x) == 0).all()
    assert sar.exp_fixed(np.float32(0.0)) == 2 ** 36
    # just above the cutoff, e·2^36 < 1/2: the fixed-point value is 0 as well,
    # so the cutoff does not change E
    assert math.exp(-25.99) * 2 ** 36 < 0.5
    assert sar.exp_fixed(np.float32(-25.99)) == 0
    # E = rint(e·2^36): compare with math.exp on a grid where e·2^36 is large
    x = np.linspace(-10, 0, 1001).astype(np.float32)
    E = sar.exp_fixed(x).astype(np.float64)
    ref = np.array([math.exp(float(t)) for t in x]) * 2.0 ** 36
    assert (np.abs(E - ref) <= 4 * 2.0 ** -24 * ref + 0.5).all()


# ---------------------------------------------------------------- quantizers

def test_pot_int8_bins_are_minimal():
    rng = np.random.default_rng(1)
    base = np.float32(0.0123)
    m = (np.exp(rng.uniform(np.log(1e-5), np.log(1e5), 20000))).astype(np.float32)
    pot = sar.pot_int8(m, base)
    b64 = float(base)
    for mv, p in zip(m[:4000], pot[:4000]):
        if p < sar.POT_HI:
            assert float(mv) <= float(np.float32(b64 * 2.0 ** p))
        if p > 0:
            assert float(mv) > float(np.float32(b64 * 2.0 ** (p - 1)))
    assert sar.pot_int8(np.float32(0.0), base) == 0
    assert sar.pot_int8(np.float32(1e30), base) == sar.POT_HI


def test_fmdq_int8_half_step_and_ceiling():
    rng = np.random.default_rng(2)
    base = np.float32(0.037)
    x = (rng.standard_normal((64, 32, 40)) * np.exp(rng.uniform(-4, 4, (1, 1, 40)))).astype(np.float32)
    x = x.reshape(64 * 32, 40)[None]                                        # [1][L][d]
    codes, pot = sar.quantize_q(x, base)
    assert np.abs(codes).max() <= sar.PCEIL8
    step = float(base) * 2.0 ** (np.repeat(pot[0], sar.SAR_TILE, axis=0) - sar.P8)
    err = np.abs(x[0].astype(np.float64) - codes[0] * step)
    assert (err <= step * (0.5 + 2.0 ** -16)).all()
    # the sub-channel maximum codes to at most the ceiling, and reaches 33..64
    tmax = np.abs(codes[0].reshape(-1, sar.SAR_TILE, 40)).max(axis=1)
    assert ((tmax >= 32) | (pot[0] == 0)).all()


def test_fmdq_int8_worked_values():
    # M = 0.7 with base 2^-4: PoT = 4 (0.5 < 0.7 ≤ 1), e = −2, step 2^-6,
    # code rint(0.7 · 64) = 45; at M = base·2^PoT exactly the code is 64.
    x = np.zeros((1, 32, 2), dtype=np.float32)
    x[0, 0, 0] = 0.7
    x[0, 5, 1] = 1.0
    codes, pot = sar.quantize_q(x, np.float32(2.0 ** -4))
    assert pot[0, 0, 0] == 4 and codes[0, 0, 0] == 45
    assert pot[0, 0, 1] == 4 and codes[0, 5, 1] == 64


def test_weight_side_int8():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((3, 128, 24)) * np.exp(rng.uniform(-3, 3, (3, 1, 24)))).astype(np.float32)
    v[1, :, 5] = 0.0
    vc, vs = sar.quantize_v(v)
    assert vs[1, 5] == 0 and (vc[1, :, 5] == 0).all()
    amax_idx = np.abs(v).argmax(axis=1)
    for b in range(3):
        for c in range(24):
            if vs[b, c] > 0:
                assert abs(vc[b, amax_idx[b, c], c]) == 127
    err = np.abs(v.astype(np.float64) - vc * vs[:, None, :].astype(np.float64))
    assert (err <= vs[:, None, :] * (0.5 + 1e-6) + 1e-30).all()
    kc, ks = sar.quantize_k(v)
    assert ks.shape == (3, 128)
    err = np.abs(v.astype(np.float64) - kc * ks[:, :, None].astype(np.float64))
    assert (err <= ks[:, :, None] * (0.5 + 1e-6) + 1e-30).all()


# ---------------------------------------------------------------- masks

def test_mask_csr_roundtrip():
    m = ga.make_mask(3, 512, 0.63, seed=5)
    row_ptr, cols = sar.mask_to_csr(m)
    back = np.zeros_like(m).reshape(-1, m.shape[2])
    for r in range(back.shape[0]):
        seg = cols[row_ptr[r]:row_ptr[r + 1]]
        assert (np.diff(seg) > 0).all()
        back[r, seg] = True
    assert (back.reshape(m.shape) == m).all()


# ---------------------------------------------------------------- closed forms

def _csr_keep(mask_rows):
    return sar.mask_to_csr(np.asarray(mask_rows, dtype=bool))


def test_uniform_attention_closed_form():
    """Q = 0: every logit is 0, P = 1/n on the kept keys (n a power of two
    here, so exactly), every P code is 64 at PoT = 15 − log2 n, and
    O = fl32(Σ_kept vq · vscale / n)."""
    L, d, heads = 512, 40, 2
    nb = L // 64
    mask = np.zeros((heads, nb, nb), dtype=bool)
    rng = np.random.default_rng(6)
    for h in range(heads):
        for qb in range(nb):
            nkeep = [1, 2, 4][(qb + h) % 3]
            mask[h, qb, rng.choice(nb, nkeep, replace=False)] = True
    row_ptr, cols = sar.mask_to_csr(mask)
    q = np.zeros((heads, L, d), dtype=np.float32)
    k = rng.standard_normal((heads, L, d)).astype(np.float32)
    v = rng.standard_normal((heads, L, d)).astype(np.float32)
    r = sar.cached_step(q, k, v, row_ptr, cols, heads, np.float32(0.01), np.float32(0.125),
                        np.float32(2.0 ** -15))
    vc, vs = sar.quantize_v(v)
    for h in range(heads):
        for qb in range(nb):
            kbs = np.nonzero(mask[h, qb])[0]
            n = 64 * len(kbs)
            j0 = row_ptr[h * nb + qb]
            for i in range(len(kbs)):
                assert (r["p"][0, j0 + i] == np.float32(1.0 / n)).all()
                assert (r["pcodes"][0, j0 + i] == 64).all()
                assert (r["ppot"][0, j0 + i] == 15 - int(math.log2(n))).all()
            keys = np.concatenate([np.arange(kb * 64, kb * 64 + 64) for kb in kbs])
            ref = (vc[h, keys].sum(axis=0).astype(np.float64) * vs[h].astype(np.float64) / n).astype(np.float32)
            got = r["o"][h, qb * 64:(qb + 1) * 64]
            assert (got == ref[None, :]).all()


def test_one_hot_attention_through_hadamard_keys():
    """K rows are Hadamard rows (orthogonal, ±1), Q[t] = 3·K[s*(t)]: the
    chosen key's logit exceeds every other (exactly 0) by more than 26, so
    P is exactly one-hot and O[t] = the quantized V row of s*(t)."""
    L, d = 128, 128
    Hm = scipy.linalg.hadamard(128).astype(np.float32)
    rng = np.random.default_rng(7)
    target = rng.integers(0, L, L)
    k = Hm[None]
    q = (3.0 * Hm[target])[None].astype(np.float32)
    v = rng.standard_normal((1, L, d)).astype(np.float32)
    row_ptr, cols = _csr_keep(np.ones((1, 2, 2)))
    r = sar.cached_step(q, k, v, row_ptr, cols, 1, np.float32(3.0 / 64), np.float32(1 / math.sqrt(d)),
                        np.float32(2.0 ** -15))
    vc, vs = sar.quantize_v(v)
    P = np.concatenate([np.concatenate([r["p"][0, 2 * qb + kb] for kb in range(2)], axis=1)
                        for qb in range(2)], axis=0)
    onehot = np.zeros((L, L), dtype=np.float32)
    onehot[np.arange(L), target] = 1.0
    assert (P == onehot).all()
    ref = (vc[0, target].astype(np.float64) * vs[0].astype(np.float64)).astype(np.float32)
    assert (r["o"][0] == ref).all()


def test_pruned_blocks_do_not_matter():
    """K and V rows of a key block that every query block prunes do not enter
    O or the cache (V changed there within its per-channel maximum elsewhere,
    so that the V scales stay the same)."""
    d = ga.make_attention(1, 2, 512, 40, 0.5, seed=8)
    mask = d["mask"].copy()
    mask[:, :, 5] = False                       # key block 5 pruned for every query block
    row_ptr, cols = sar.mask_to_csr(mask)
    args = (row_ptr, cols, 2, d["base_q"], d["sm_scale"], d["base_p"])
    rng = np.random.default_rng(9)
    blk = np.s_[:, 320:384]
    amax_out = np.abs(np.delete(d["v"], np.s_[320:384], axis=1)).max(axis=1)[:, None, :]
    va, vb = d["v"].copy(), d["v"].copy()
    va[blk] = (rng.uniform(-0.5, 0.5, (2, 64, 40)) * amax_out).astype(np.float32)
    vb[blk] = (rng.uniform(-0.5, 0.5, (2, 64, 40)) * amax_out).astype(np.float32)
    kb = d["k"].copy()
    kb[blk] = (rng.standard_normal((2, 64, 40)) * 100).astype(np.float32)
    assert (sar.quantize_v(va)[1] == sar.quantize_v(vb)[1]).all()
    a = sar.cached_step(d["q"], d["k"], va, *args)
    b = sar.cached_step(d["q"], kb, vb, *args)
    assert (a["o"] == b["o"]).all()
    assert (a["pcodes"] == b["pcodes"]).all() and (a["ppot"] == b["ppot"]).all()


# ---------------------------------------------------------------- brute force

def test_brute_force_tiny():
    """Pure-Python integers for the scores and outputs, math.exp softmax in
    float64: exact integer scores, P within 2^-20 (relative to the row
    maximum) and O equal to the float64 product of the oracle's own quantized
    P and V within one float32 rounding."""
    dd = ga.make_attention(1, 1, 128, 8, 0.8, seed=10)
    mask = np.array([[[True, False], [True, True]]])
    row_ptr, cols = sar.mask_to_csr(mask)
    r = sar.cached_step(dd["q"], dd["k"], dd["v"], row_ptr, cols, 1, dd["base_q"], dd["sm_scale"], dd["base_p"])
    qc, qp, kc, ks = r["qcodes"][0], r["qpot"][0], r["kcodes"][0], r["kscale"][0]
    g = float(dd["base_q"]) * 2.0 ** -6 * float(dd["sm_scale"])
    blocks = [(0, 0), (1, 0), (1, 1)]
    for j, (qb, kb) in enumerate(blocks):
        for t in range(64):
            row = qb * 64 + t
            kept = [kk for (qq, kk) in blocks if qq == qb]
            keys = [kk * 64 + s for kk in kept for s in range(64)]
            z = {}
            for s in keys:
                acc = 0
                for c in range(8):
                    acc += int(qc[row, c]) * (1 << int(qp[row // 32, c])) * int(kc[s, c])
                z[s] = acc * (float(ks[s]) * g)
            m = max(z.values())
            den = sum(math.exp(z[s] - m) for s in keys)
            for s in range(64):
                p = math.exp(z[kb * 64 + s] - m) / den
                assert abs(float(r["p"][0, j, t, s]) - p) <= 2.0 ** -20 * max(1.0, p)
    # O from the oracle's own quantized P and V, in float64 by loops
    vc, vs = r["vcodes"][0], r["vscale"][0]
    for row in range(0, 128, 7):
        qb = row // 64
        t = row % 64
        for c in range(8):
            acc = 0
            for j, (qq, kb) in enumerate(blocks):
                if qq != qb:
                    continue
                for s in range(64):
                    acc += int(r["pcodes"][0, j, t, s]) * (1 << int(r["ppot"][0, j, t // 32, s])) * int(vc[kb * 64 + s, c])
            ref = float(np.float32(acc * float(vs[c]) * float(dd["base_p"]) * 2.0 ** -6))
            assert abs(float(r["o"][0, row, c]) - ref) <= 2.0 ** -23 * abs(ref) + 1e-30


def test_close_to_float64_masked_attention():
    """The quantized path approximates plain masked softmax attention: the
    error of O stays within a few percent of max |V| (8-bit operands)."""
    dd = ga.make_attention(1, 2, 256, 72, 0.63, seed=11)
    row_ptr, cols = sar.mask_to_csr(dd["mask"])
    r = sar.cached_step(dd["q"], dd["k"], dd["v"], row_ptr, cols, 2, dd["base_q"], dd["sm_scale"], dd["base_p"])
    for h in range(2):
        q = dd["q"][h].astype(np.float64)
        k = dd["k"][h].astype(np.float64)
        v = dd["v"][h].astype(np.float64)
        z = q @ k.T / math.sqrt(72)
        keep = np.kron(dd["mask"][h], np.ones((64, 64), dtype=bool))
        z = np.where(keep, z, -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ v
        assert np.abs(r["o"][h] - o).max() <= 0.03 * np.abs(v).max()


def test_rows_sum_to_one_and_reuse_with_same_v():
    dd = ga.make_attention(2, 2, 256, 72, 0.63, seed=12)
    row_ptr, cols = sar.mask_to_csr(dd["mask"])
    r = sar.cached_step(dd["q"], dd["k"], dd["v"], row_ptr, cols, 2, dd["base_q"], dd["sm_scale"], dd["base_p"])
    nb = 4
    for b in range(2):
        for h in range(2):
            for qb in range(nb):
                j0, j1 = row_ptr[h * nb + qb], row_ptr[h * nb + qb + 1]
                s = r["p"][b, j0:j1].astype(np.float64).sum(axis=(0, 2))
                assert np.abs(s - 1).max() <= 2.0 ** -18
    u = sar.reused_step(r["pcodes"], r["ppot"], dd["v"], row_ptr, cols, 2, dd["base_p"])
    assert (u["o"] == r["o"]).all()
    u2 = sar.reused_step(r["pcodes"], r["ppot"], dd["v_next"], row_ptr, cols, 2, dd["base_p"])
    assert not (u2["o"] == r["o"]).all()
