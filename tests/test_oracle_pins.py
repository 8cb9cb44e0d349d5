"""Pins of the CPU oracle against facts it does not derive from itself.

Every test here ties a part of ``oracle/fmdq.py`` to something fixed outside
the oracle: values printed in DSTAR (arXiv 2607.15846; fixtures under
``tests/golden/``), closed forms, library routines, exact rational arithmetic
or brute force.  A dropped term, a wrong sign, a wrong index or a transposed
operand anywhere in the oracle fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from gen import workloads as wl
from oracle import fmdq
from tests import digits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dstar_examples.json")
with open(GOLDEN) as f:
    EX = json.load(f)


# ------------------------------------------------------------------ P1 -------
def test_worked_example_section_3_1():
    """DSTAR §3.1 ❶ worked example: M=0.7, base=2^-4, 2-bit threshold 2^0
    → 2-bit, PCeil=1, PoT=4, FPoT=4, s=1."""
    ex = EX["worked_example"]
    base = ex["base"]
    k0 = int(round(math.log2(ex["thr_2bit"] / base)))
    assert k0 == 4
    m = np.array([ex["M"]], dtype=np.float32)
    pot = fmdq.pot_exponent(m, base)
    bits = fmdq.precision_bits(pot, k0)
    tag = fmdq.fpot_tag(bits, pot)
    assert int(pot[0]) == ex["PoT"]
    assert int(bits[0]) == ex["bits"]
    assert fmdq.PCEIL[int(bits[0])] == ex["PCeil"]
    # Eq. 4 FPoT = tag − 15 − 2·log2(base) for a power-of-two base.
    assert int(tag[0]) - fmdq.TAG_OFF - 2 * int(math.log2(base)) == ex["FPoT"]
    # Eq. 5 s = base·2^FPoT; the step 1/s = base·2^e.
    e = int(fmdq.step_exponent(tag)[0])
    assert 1.0 / (base * 2.0 ** e) == ex["s"]
    # The value itself lands on code 1 (0.7·s = 0.7 rounds to 1, within PCeil).
    q = fmdq.quantize_values(m, np.array([e]), bits, fmdq.inv_base_f32(base))
    assert int(q[0]) == 1


# ------------------------------------------------------------------ P2 -------
@pytest.mark.parametrize("log2_base", [-8, -4, -1, 0, 3])
def test_eq2_equals_eq5_for_power_of_two_base(log2_base):
    """Eq. 2 (s = PCeil/(base·2^PoT)) and Eq. 5 (s = base·2^FPoT with Eq. 4's
    FPoT) give the same scale; the oracle's step 2^e·base is 1/s."""
    base = 2.0 ** log2_base
    rng = np.random.default_rng(7)
    m = (np.exp(rng.uniform(np.log(base * 1e-3), np.log(base * 2.0 ** 20), 4000))).astype(np.float32)
    for k0 in (1, 2, 4, 9):
        pot = fmdq.pot_exponent(m, base)
        bits = fmdq.precision_bits(pot, k0)
        tag = fmdq.fpot_tag(bits, pot)
        e = fmdq.step_exponent(tag)
        for i in range(0, len(m), 97):
            pceil = fmdq.PCEIL[int(bits[i])]
            s_eq2 = pceil / (base * 2.0 ** int(pot[i]))
            fpot = math.log2(pceil / (base * base * 2.0 ** int(pot[i])))  # Eq. 4
            s_eq5 = base * 2.0 ** fpot
            assert s_eq2 == s_eq5
            assert s_eq2 == 1.0 / (base * 2.0 ** int(e[i]))
            assert 0 <= int(tag[i]) <= 15


# ------------------------------------------------------------------ P3 -------
def test_slice_shift_example_section_3_1():
    """DSTAR §3.1 ❷: 70 = slices 1,0,1,2 with FPoT 1,3,5,7; accumulating in
    ascending FPoT with left shifts by the FPoT difference gives 70·w.  The
    oracle's shift_combine must give the same with the FPoTs mapped to tags."""
    ex = EX["slice_example"]
    slices, fpots = ex["slices_hi_to_lo"], ex["fpot_hi_to_lo"]
    assert sum(s << (2 * (3 - i)) for i, s in enumerate(slices)) == ex["value"]
    w = np.array([[3, -7, 11]], dtype=np.int64)
    # The page's own procedure: ascending FPoT, shift left by ΔFPoT each step.
    order = np.argsort(fpots)
    psum = np.zeros_like(w)
    prev = None
    for i in order:
        if prev is not None:
            assert fpots[i] - prev >= 0
            psum = psum << (fpots[i] - prev)
        psum = psum + slices[i] * w
        prev = fpots[i]
    assert fpots[order[1]] - fpots[order[0]] == ex["first_shift"]
    np.testing.assert_array_equal(psum, ex["value"] * w)
    # The oracle: tags = FPoT + 8 (any constant offset keeps FPoT differences).
    acc = np.zeros((16, 1, 3), dtype=np.int64)
    for s, fp in zip(slices, fpots):
        acc[fp + 8] += s * w
    np.testing.assert_array_equal(fmdq.shift_combine(acc), ex["value"] * w)


def test_shift_combine_equals_horner_in_ascending_fpot():
    """Random group sums: the closed form Σ acc_g·2^(15−g) equals the page's
    Horner accumulation (ascending FPoT = ascending tag, left shift by the tag
    difference, final shift to the tag-15 unit)."""
    rng = np.random.default_rng(3)
    for _ in range(50):
        acc = np.zeros((16, 2, 5), dtype=np.int64)
        present = rng.choice(16, size=rng.integers(1, 9), replace=False)
        for g in present:
            acc[g] = rng.integers(-2**30, 2**30, size=(2, 5))
        tags = sorted(present)
        h = np.zeros((2, 5), dtype=np.int64)
        prev = tags[0]
        for g in tags:
            h = (h << (g - prev)) + acc[g]
            prev = g
        h = h << (15 - tags[-1])
        np.testing.assert_array_equal(fmdq.shift_combine(acc), h)


# ------------------------------------------------------------------ P4 -------
@pytest.mark.parametrize("rows,T", [(96, 32), (70, 32), (64, 64), (40, 16)])
def test_zero_delta_returns_cached_output_exactly(rows, T):
    """Eq. 1 with Δx = 0: y' = y, bit for bit."""
    d = wl.make_custom(rows, 40, 24, T, seed=11, zero_delta=True)
    r = fmdq.layer(d["x_t"], d["x_prev"], d["w"], d["w_scale"], d["y_prev"],
                   d["base"], T, d["k0"])
    assert not r["codes"].any()
    np.testing.assert_array_equal(r["y"], d["y_prev"])
    assert (fmdq.bits_of(r["tags"]) == 2).all()


# ------------------------------------------------------------------ P5 -------
def test_pot_is_minimal_power_of_two_bin_and_matches_ceil_log2():
    rng = np.random.default_rng(5)
    base = 0.0371
    m = np.exp(rng.uniform(np.log(base / 50), np.log(base * 2 ** 23), 20000)).astype(np.float32)
    pot = fmdq.pot_exponent(m, base)
    b32 = np.float32(base)
    for x, p in zip(m[:3000], pot[:3000]):
        x, p = float(x), int(p)
        if x <= float(b32):
            assert p == 0
        elif x > float(b32) * 2.0 ** fmdq.POT_HI:
            assert p == fmdq.POT_HI
        else:
            # closed form of Eq. 3 away from the bin edges
            ratio = x / float(b32)
            if abs(math.log2(ratio) - round(math.log2(ratio))) > 1e-6:
                assert p == math.ceil(math.log2(ratio))
            assert float(b32) * 2.0 ** (p - 1) < x <= float(b32) * 2.0 ** p
    # exact bin edges belong to the lower bin (closed upper edge)
    edges = np.array([b32 * np.float32(2.0 ** j) for j in range(0, 22)], dtype=np.float32)
    np.testing.assert_array_equal(fmdq.pot_exponent(edges, base), np.arange(22))
    above = np.nextafter(edges, np.float32(np.inf))
    np.testing.assert_array_equal(fmdq.pot_exponent(above[:-1], base), np.arange(1, 22))


def test_precision_from_thresholds_thr0_times_4_to_the_n():
    """DSTAR §3.1 ❶: bits from binning M against Thr_N = Thr_0·2^(2N)."""
    rng = np.random.default_rng(9)
    base = 0.02
    b32 = float(np.float32(base))
    m = np.exp(rng.uniform(np.log(base / 10), np.log(base * 2 ** 20), 20000)).astype(np.float32)
    for k0 in (1, 2, 3, 4, 7):
        thr0 = b32 * 2.0 ** k0
        expect = np.full(m.shape, 8)
        for n, b in ((2, 6), (1, 4), (0, 2)):
            expect = np.where(m.astype(np.float64) <= thr0 * 4.0 ** n, b, expect)
        got = fmdq.precision_bits(fmdq.pot_exponent(m, base), k0)
        np.testing.assert_array_equal(got, expect)


def _layer_with_internals(d):
    delta = fmdq.differential(d["x_t"], d["x_prev"])
    r = fmdq.layer(d["x_t"], d["x_prev"], d["w"], d["w_scale"], d["y_prev"],
                   d["base"], d["token_tile"], d["k0"])
    return delta, r


@pytest.mark.parametrize("seed,rows,K,T,heavy", [
    (1, 96, 48, 32, 0.03), (2, 70, 33, 32, 0.2), (3, 128, 20, 64, 0.5), (4, 50, 17, 16, 0.1)])
def test_codes_within_pceil_and_half_step(seed, rows, K, T, heavy):
    """|q| ≤ PCeil of the sub-channel; |Δ − q·δ| ≤ δ·(1/2 + 2^−16) (the two
    float32 roundings of the code path at |r| ≤ 64)."""
    d = wl.make_custom(rows, K, 8, T, seed=seed, heavy=heavy)
    delta, r = _layer_with_internals(d)
    codes, tags = r["codes"], r["tags"]
    bits = fmdq.bits_of(tags)
    e = fmdq.step_exponent(fmdq.tag_of(tags))
    b32 = float(np.float32(d["base"]))
    for tau in range(codes.shape[0]):
        r0, r1 = fmdq.tile_rows(tau, rows, T)
        assert not codes[tau, :, r1 - r0:].any(), "padded rows must be zero"
        for k in range(K):
            pc = fmdq.PCEIL[int(bits[tau, k])]
            q = codes[tau, k, : r1 - r0].astype(np.int64)
            assert np.abs(q).max() <= pc
            step = b32 * 2.0 ** int(e[tau, k])
            err = np.abs(delta[r0:r1, k].astype(np.float64) - q * step)
            assert err.max() <= step * (0.5 + 2.0 ** -16)
            # the sub-channel's largest value uses the full range of its precision
            m = float(np.abs(delta[r0:r1, k]).max())
            if m > b32:
                assert np.abs(q).max() >= pc // 2


def test_saturated_subchannel_clips_at_pceil():
    base = 0.01
    rows, K, T = 32, 4, 32
    x_prev = np.zeros((rows, K), dtype=np.float32)
    x_t = np.zeros((rows, K), dtype=np.float32)
    x_t[3, 1] = np.float32(base * 2.0 ** 23)      # above base·2^POT_HI
    x_t[5, 1] = np.float32(-base * 2.0 ** 19)
    codes, tags, hist = fmdq.quantize(x_t, x_prev, T, base, 2)
    assert int(fmdq.bits_of(tags)[0, 1]) == 8
    assert int(fmdq.tag_of(tags)[0, 1]) == 0      # PoT 21, e = 15
    assert codes[0, 1, 3] == 64 and codes[0, 1, 5] == -16
    np.testing.assert_array_equal(hist, [3, 0, 0, 1])


# ------------------------------------------------------------------ P7 -------
@pytest.mark.parametrize("seed,rows,K,N,T", [(21, 96, 64, 40, 32), (22, 45, 37, 9, 16), (23, 128, 50, 12, 64)])
def test_shift_aligned_equals_dequantize_then_multiply(seed, rows, K, N, T):
    """Grouped sums aligned by shifts == one plain integer GEMM of the
    dequantized codes in natural channel order (codes · 2^e, no grouping)."""
    d = wl.make_custom(rows, K, N, T, seed=seed, heavy=0.2)
    codes, tags, _ = fmdq.quantize(d["x_t"], d["x_prev"], T, d["base"], d["k0"])
    perm, off = fmdq.bucket(tags)
    e = fmdq.step_exponent(fmdq.tag_of(tags))
    w = d["w"].astype(np.int64)
    for tau in range(codes.shape[0]):
        acc = fmdq.group_accumulators(codes[tau], perm[tau], off[tau], d["w"])
        s = fmdq.shift_combine(acc)
        scaled = codes[tau].T.astype(np.int64) * (np.int64(1) << e[tau].astype(np.int64))[None, :]
        np.testing.assert_array_equal(s, np.matmul(scaled, w))
        # each group sum equals the masked natural-order product
        for g in range(16):
            mask = (fmdq.tag_of(tags[tau]) == g)
            ref = np.matmul(codes[tau].T.astype(np.int64) * mask[None, :], w)
            np.testing.assert_array_equal(acc[g], ref)


# ------------------------------------------------------------------ P8 -------
def _brute_force_layer(d):
    """Pure-Python, element-by-element FMDQ layer with exact rational output."""
    rows, K = d["x_t"].shape
    N = d["w"].shape[1]
    T, k0 = d["token_tile"], d["k0"]
    f32 = np.float32
    b32 = f32(d["base"])
    inv = f32(1.0 / float(b32))
    nt = (rows + T - 1) // T
    deq = [[Fraction(0)] * K for _ in range(rows)]
    codes = {}
    for tau in range(nt):
        rs = range(tau * T, min(rows, tau * T + T))
        for k in range(K):
            dl = [f32(f32(d["x_t"][r, k]) - f32(d["x_prev"][r, k])) for r in rs]
            m = max(abs(float(v)) for v in dl)
            pot = next((j for j in range(22) if m <= float(b32) * 2.0 ** j), 21)
            bits = 2 if pot <= k0 else 4 if pot <= k0 + 2 else 6 if pot <= k0 + 4 else 8
            pc = 2 ** (bits - 2)
            e = pot - (bits - 2)
            for r, v in zip(rs, dl):
                x = f32(f32(v * inv) * f32(2.0 ** -e))
                q = int(np.rint(x))
                q = max(-pc, min(pc, q))
                codes[(r, k)] = q
                deq[r][k] = Fraction(q) * Fraction(float(b32)) * Fraction(2) ** e
    y = np.zeros((rows, N), dtype=np.float32)
    exact = [[None] * N for _ in range(rows)]
    for r in range(rows):
        for n in range(N):
            acc = sum(deq[r][k] * int(d["w"][k, n]) for k in range(K))
            v = Fraction(float(d["y_prev"][r, n])) + acc * Fraction(float(d["w_scale"][n]))
            exact[r][n] = v
            y[r, n] = np.float32(float(v))
    return codes, y, exact


@pytest.mark.parametrize("seed,rows,K,N,T,heavy", [
    (31, 40, 12, 5, 16, 0.2), (32, 70, 9, 4, 32, 0.3), (33, 33, 20, 3, 32, 0.05), (34, 64, 7, 6, 64, 0.5)])
def test_brute_force_tiny_layers(seed, rows, K, N, T, heavy):
    """Whole layer against an element-by-element implementation with exact
    rational arithmetic: codes identical, Y within one float32 ulp of the exact
    value rounded to float32 (the oracle rounds in float64 first)."""
    d = wl.make_custom(rows, K, N, T, seed=seed, heavy=heavy)
    r = fmdq.layer(d["x_t"], d["x_prev"], d["w"], d["w_scale"], d["y_prev"], d["base"], T, d["k0"])
    codes, y_bf, _ = _brute_force_layer(d)
    for (row, k), q in codes.items():
        assert r["codes"][row // T, k, row % T] == q
    ulp = np.spacing(np.abs(y_bf).astype(np.float32))
    assert (np.abs(r["y"].astype(np.float64) - y_bf) <= ulp).all()


# ------------------------------------------------------------------ P9 -------
def test_single_group_reduces_to_plain_int8_gemm():
    """All sub-channels share one M → one tag → S is a plain int GEMM of the
    codes times 2^e, Y = Y_prev + w_scale·base·2^e·(Q @ W)."""
    rng = np.random.default_rng(41)
    rows, K, N, T = 96, 24, 10, 32
    base = 0.05
    x_prev = rng.standard_normal((rows, K)).astype(np.float32)
    delta = rng.uniform(-0.9, 0.9, (rows, K)) * 0.37
    for tau in range(rows // T):
        delta[tau * T, :] = 0.37                      # same maximum everywhere
    x_t = (x_prev.astype(np.float64) + delta).astype(np.float32)
    dd = fmdq.differential(x_t, x_prev)
    m = fmdq.subchannel_max(dd, T)
    # the fp32 subtraction may move the maximum by an ulp: force equal bins
    assert len(np.unique(fmdq.pot_exponent(m, base))) == 1
    w = rng.integers(-127, 128, (K, N)).astype(np.int8)
    ws = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    y0 = rng.standard_normal((rows, N)).astype(np.float32)
    r = fmdq.layer(x_t, x_prev, w, ws, y0, base, T, 2)
    tg = np.unique(fmdq.tag_of(r["tags"]))
    assert len(tg) == 1
    e = 15 - int(tg[0])
    q = r["codes"].transpose(0, 2, 1).reshape(rows, K).astype(np.int64)
    s = np.matmul(q, w.astype(np.int64)) << e
    expect = (y0.astype(np.float64) + (s.astype(np.float64) * float(np.float32(base))) * ws.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(r["y"], expect)


# ------------------------------------------------------------------ P10 ------
def test_exact_grid_input_roundtrips_and_gives_closed_form_output():
    """Δ built on the quantization grid (Δ = q·base·2^e, each sub-channel
    hitting its bin edge): codes == q exactly, and Y == fl32(Y_prev +
    w_scale·(Δ @ W)) with Δ @ W exact in float64."""
    rng = np.random.default_rng(51)
    rows, K, N, T, k0 = 64, 30, 7, 32, 2
    base = 2.0 ** -5
    x_prev = np.zeros((rows, K), dtype=np.float32)
    x_t = np.zeros((rows, K), dtype=np.float32)
    qs = np.zeros((rows, K), dtype=np.int64)
    for tau in range(rows // T):
        for k in range(K):
            bits = int(rng.choice([2, 4, 6, 8]))
            pc = 2 ** (bits - 2)
            pot = {2: rng.integers(0, k0 + 1), 4: rng.integers(k0 + 1, k0 + 3),
                   6: rng.integers(k0 + 3, k0 + 5), 8: rng.integers(k0 + 5, 22)}[bits]
            e = int(pot) - (bits - 2)
            q = rng.integers(-pc, pc + 1, T)
            q[rng.integers(0, T)] = pc * int(rng.choice([-1, 1]))   # reach the bin edge
            if pot == 0:
                q[:] = np.clip(q, -1, 1)
            qs[tau * T:(tau + 1) * T, k] = q
            x_t[tau * T:(tau + 1) * T, k] = (q * base * 2.0 ** e).astype(np.float32)
    w = rng.integers(-127, 128, (K, N)).astype(np.int8)
    ws = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    y0 = rng.standard_normal((rows, N)).astype(np.float32)
    r = fmdq.layer(x_t, x_prev, w, ws, y0, base, T, k0)
    got = r["codes"].transpose(0, 2, 1).reshape(rows, K).astype(np.int64)
    np.testing.assert_array_equal(got, qs)
    dw = np.matmul(x_t.astype(np.float64), w.astype(np.float64))
    expect = (y0.astype(np.float64) + dw * ws.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(r["y"], expect)


# ------------------------------------------------------------------ P11 ------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bucket_is_stable_sort_and_max_is_abs_max(seed):
    rng = np.random.default_rng(seed)
    nt, K = 6, 301
    raw = rng.integers(0, 16, (nt, K)) | (rng.integers(0, 4, (nt, K)) << 4)
    tags = raw.astype(np.uint8)
    perm, off = fmdq.bucket(tags)
    for tau in range(nt):
        tg = (tags[tau] & 0x0F).astype(np.int64)
        pc = ((tags[tau] >> 4) & 0x3).astype(np.int64)
        # the library routine on the same key: tag ascending, precision descending
        key = np.lexsort((3 - pc, tg))       # last key is primary; lexsort is stable
        np.testing.assert_array_equal(perm[tau], key)
        bins = 4 * tg + 3 - pc
        np.testing.assert_array_equal(off[tau], np.concatenate([[0], np.cumsum(np.bincount(bins, minlength=64))]))
        # FPoT groups are contiguous and ascending; inside a group the precision
        # never increases and, at equal precision, channel ids increase
        t_sorted, p_sorted = tg[perm[tau]], pc[perm[tau]]
        assert (np.diff(t_sorted) >= 0).all()
        for g in range(16):
            lo, hi = fmdq.group_bounds(off[tau], g)
            assert (t_sorted[lo:hi] == g).all() and hi - lo == int((tg == g).sum())
            assert (np.diff(p_sorted[lo:hi]) <= 0).all()
            same = np.diff(p_sorted[lo:hi]) == 0
            assert (np.diff(perm[tau][lo:hi].astype(int))[same] > 0).all()
    d = rng.standard_normal((70, 13)).astype(np.float32)
    m = fmdq.subchannel_max(d, 32)
    pad = np.zeros((96, 13), dtype=np.float32)
    pad[:70] = np.abs(d)
    np.testing.assert_array_equal(m, pad.reshape(3, 32, 13).max(axis=1))


# ------------------------------------------------------------------ P12 ------
def test_fig11_meta_table_order():
    """Fig. 11: meta items stream in ascending FPoT (ties in any order).  The
    bucket of the same items, shuffled, yields the same FPoT column."""
    t = EX["fig11_meta_table"]
    fp = np.array(t["fpot"])
    assert (np.diff(fp) >= 0).all()
    rng = np.random.default_rng(0)
    sh = rng.permutation(len(fp))
    tags = fp[sh].astype(np.uint8)[None, :]
    perm, off = fmdq.bucket(tags)
    np.testing.assert_array_equal(fp[sh][perm[0].astype(int)], fp)
    # items of one FPoT keep their relative (stable) order
    for g in np.unique(fp):
        lo, hi = fmdq.group_bounds(off[0], int(g))
        idx = perm[0][lo:hi]
        assert (np.diff(idx.astype(int)) > 0).all()


def test_differential_is_float32_subtraction():
    a = np.array([[1.0, 1e8, -3.5]], dtype=np.float32)
    b = np.array([[np.nextafter(np.float32(1.0), np.float32(2.0)), 1e8 + 4, 2.25]], dtype=np.float32)
    np.testing.assert_array_equal(fmdq.differential(a, b), (a - b))
    assert fmdq.differential(a, b).dtype == np.float32


def test_code_rounding_is_half_to_even():
    """The pages do not fix the rounding of codes; the reading is IEEE
    round-half-to-even (Python's round()).  Exact ties decide it."""
    base, T, k0 = 2.0 ** -4, 32, 2
    x_prev = np.zeros((T, 1), dtype=np.float32)
    halves = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5, 4.0] + [0.0] * (T - 9))
    x_t = (halves * base * 2.0 ** 2)[:, None].astype(np.float32)   # step base·2^2 (4-bit, PoT 4)
    codes, tags, _ = fmdq.quantize(x_t, x_prev, T, base, k0)
    assert int(fmdq.bits_of(tags)[0, 0]) == 4 and int(fmdq.step_exponent(fmdq.tag_of(tags))[0, 0]) == 2
    np.testing.assert_array_equal(codes[0, 0, :9], [round(v) for v in halves[:9]])


# ------------------------------------------------------------------ P13 ------
def test_code_digits_reconstruct_every_shift_aligned_code():
    """a = d0 + 2^7·d1 + 2^15·d2 for every value a code can take in units of
    the base (|q·2^e| ≤ 2^PoT ≤ 2^21), with every digit in 8 bits, and no third
    digit while |a| ≤ 2^13 (brute force over the whole range)."""
    a = np.arange(-(1 << 21), (1 << 21) + 1, dtype=np.int64)
    d0, d1, d2 = digits.code_digits(a)
    np.testing.assert_array_equal(d0 + 128 * d1 + 32768 * d2, a)
    assert d0.min() == -64 and d0.max() == 63
    assert d1.min() >= -128 and d1.max() <= 127
    assert d2.min() >= -64 and d2.max() <= 64
    small = np.abs(a) <= (1 << 13)
    assert not d2[small].any() and np.abs(d1[small]).max() <= 64
    # a few values by hand: 64 = -64 + 2^7; 2^21 = 64·2^15; -65 = 63 - 2^7
    for v, want in ((64, (-64, 1, 0)), (1 << 21, (0, 0, 64)), (-65, (63, -1, 0)), (-1, (-1, 0, 0))):
        got = tuple(int(x[0]) for x in digits.code_digits(np.array([v])))
        assert got == want, (v, got)


@pytest.mark.parametrize("seed,rows,K,N,T,c_range", [(31, 96, 64, 24, 32, (0.5, 64.0)),
                                                     (32, 70, 40, 8, 32, (0.5, 64.0)),
                                                     (33, 128, 36, 12, 64, (0.5, 64.0)),
                                                     (34, 64, 48, 16, 32, (0.02, 4000.0))])
def test_aligned_codes_and_digit_planes_split_S_exactly(seed, rows, K, N, T, c_range):
    """S = A·W + 2^7·(D1·W) + 2^15·(D2·W) per tile, exactly, against the
    per-FPoT-group sum; A = q·2^e where PoT ≤ 6; digit planes zero where the
    sub-channel does not need them."""
    d = wl.make_custom(rows, K, N, T, seed=seed, heavy=0.3, c_range=c_range)
    codes, tags, _ = fmdq.quantize(d["x_t"], d["x_prev"], T, d["base"], d["k0"])
    a = digits.aligned_codes(codes, tags)
    h = digits.heavy_digits(codes, tags)
    nt = codes.shape[0]
    assert a.shape == (nt * T, K) and a.dtype == np.int8
    assert h.shape == (2, nt, K, T) and h.dtype == np.int8
    e = fmdq.step_exponent(fmdq.tag_of(tags))
    pot = e + fmdq.bits_of(tags) - 2
    assert (pot > 6).any() and (pot <= 6).any()
    if c_range[1] > 1000:
        assert (pot > 13).any()          # the third digit is exercised
    perm, off = fmdq.bucket(tags)
    w = d["w"].astype(np.int64)
    for tau in range(nt):
        at = a[tau * T:(tau + 1) * T].astype(np.int64)                     # [T][K]
        qt = codes[tau].T.astype(np.int64)                                   # [T][K]
        light = pot[tau] <= 6
        np.testing.assert_array_equal(at[:, light], qt[:, light] << e[tau][light])
        d1 = h[0, tau].T.astype(np.int64)
        d2 = h[1, tau].T.astype(np.int64)
        np.testing.assert_array_equal(d1[:, light], 0)
        np.testing.assert_array_equal(d2[:, pot[tau] <= 13], 0)
        s = fmdq.shift_combine(fmdq.group_accumulators(codes[tau], perm[tau], off[tau], d["w"]))
        np.testing.assert_array_equal(at @ w + 128 * (d1 @ w) + 32768 * (d2 @ w), s)