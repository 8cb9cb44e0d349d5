"""Pins of the oracle's dynamic base (DSTAR §3.1 ❶: the base is the smallest
sub-channel maximum M_i of the layer input; §5.2 Table 2 "DS-FMDQ-DYN").

The base is checked against facts fixed outside ``oracle.fmdq``: the defining
properties of a minimum over sub-channel maxima computed here with a different
formulation (reshape + reduce instead of the oracle's row loop), Eq. 2/3 in
exact rational arithmetic at the minimum, exact equivariance under power-of-two
scaling of the input, and the special cases (zero sub-channels, clamping).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from gen import workloads as wl
from oracle import fmdq


def subchannel_max_reshape(x_t, x_prev, T):
    """M_{τk} by padding the rows to whole tiles with Δ = 0 and reducing."""
    d = np.abs(np.subtract(x_t.astype(np.float32), x_prev.astype(np.float32), dtype=np.float32))
    rows, K = d.shape
    nt = -(-rows // T)
    pad = np.zeros((nt * T, K), dtype=np.float32)
    pad[:rows] = d
    return pad.reshape(nt, T, K).max(axis=1)


CASES = [(96, 40, 32, 1), (70, 24, 32, 2), (128, 36, 64, 3), (40, 17, 16, 4), (1, 5, 32, 5)]


@pytest.mark.parametrize("rows,K,T,seed", CASES)
def test_base_is_the_smallest_positive_subchannel_max(rows, K, T, seed):
    d = wl.make_custom(rows, K, 8, T, seed=seed)
    b = fmdq.dynamic_base(d["x_t"], d["x_prev"], T, d["base"])
    m = subchannel_max_reshape(d["x_t"], d["x_prev"], T)
    pos = m[m > 0]
    assert isinstance(b, np.float32)
    assert (pos >= b).all()               # no positive sub-channel maximum below the base
    assert (pos == b).any()               # and the base is one of them


@pytest.mark.parametrize("rows,K,T,seed", CASES[:4])
def test_subchannel_at_the_minimum_has_pot_0_and_unit_code(rows, K, T, seed):
    """Eq. 3 gives PoT = ⌈log2(M/base)⌉ ≥ 0 for every sub-channel (the floor is
    never needed), = 0 at the minimum, whose largest |Δ| is coded ±PCeil = ±1
    (Eq. 2: s = 1/base)."""
    d = wl.make_custom(rows, K, 8, T, seed=seed)
    b = fmdq.dynamic_base(d["x_t"], d["x_prev"], T, d["base"])
    codes, tags, _ = fmdq.quantize(d["x_t"], d["x_prev"], T, b, d["k0"])
    m = subchannel_max_reshape(d["x_t"], d["x_prev"], T)
    pot = fmdq.step_exponent(fmdq.tag_of(tags)) + fmdq.bits_of(tags) - 2
    fb = Fraction(float(b))
    for tau in range(m.shape[0]):
        for k in range(K):
            if m[tau, k] == 0:
                continue
            r = Fraction(float(m[tau, k])) / fb
            j = 0
            while Fraction(2) ** j < r:
                j += 1
            assert pot[tau, k] == min(j, fmdq.POT_HI)
    at_min = np.argwhere(m == b)
    assert len(at_min)
    delta = fmdq.differential(d["x_t"], d["x_prev"])
    for tau, k in at_min:
        assert pot[tau, k] == 0 and fmdq.bits_of(tags)[tau, k] == 2
        r0, r1 = tau * T, min(tau * T + T, rows)
        col = delta[r0:r1, k]
        t = int(np.argmax(np.abs(col)))
        assert codes[tau, k, t] == int(np.sign(col[t]))


@pytest.mark.parametrize("s", [5, -7, 20])
def test_power_of_two_scaling_scales_the_base_and_keeps_the_codes(s):
    d = wl.make_custom(70, 24, 16, 32, seed=9)
    f = np.float32(2.0 ** s)
    x_t, x_p = d["x_t"] * f, d["x_prev"] * f             # exact in float32
    b0 = fmdq.dynamic_base(d["x_t"], d["x_prev"], 32, d["base"])
    b1 = fmdq.dynamic_base(x_t, x_p, 32, d["base"])
    assert b1 == np.float32(math.ldexp(float(b0), s))
    y0 = np.zeros_like(d["y_prev"])
    r0 = fmdq.layer_dynamic(d["x_t"], d["x_prev"], d["w"], d["w_scale"], y0, d["base"], 32, d["k0"])
    r1 = fmdq.layer_dynamic(x_t, x_p, d["w"], d["w_scale"], y0, d["base"], 32, d["k0"])
    np.testing.assert_array_equal(r1["codes"], r0["codes"])
    np.testing.assert_array_equal(r1["tags"], r0["tags"])
    np.testing.assert_array_equal(r1["y"], (r0["y"].astype(np.float64) * 2.0 ** s).astype(np.float32))


def test_zero_subchannels_are_left_out_and_all_zero_keeps_the_static_base():
    d = wl.make_custom(64, 12, 8, 32, seed=12)
    x_t = d["x_t"].copy()
    x_t[32:64, 3] = d["x_prev"][32:64, 3]                # sub-channel (1, 3): Δ = 0
    b = fmdq.dynamic_base(x_t, d["x_prev"], 32, d["base"])
    m = subchannel_max_reshape(x_t, d["x_prev"], 32)
    assert m[1, 3] == 0 and b > 0 and b == m[m > 0].min()
    z = fmdq.dynamic_base(d["x_prev"], d["x_prev"], 32, d["base"])
    assert z == np.float32(d["base"])


def test_sign_of_delta_does_not_matter():
    """M is a maximum of |Δ|: negating Δ (swapping X_t and X_{t−1}) keeps the base."""
    d = wl.make_custom(70, 24, 8, 32, seed=13)
    assert fmdq.dynamic_base(d["x_t"], d["x_prev"], 32, 1.0) == fmdq.dynamic_base(d["x_prev"], d["x_t"], 32, 1.0)


@pytest.mark.parametrize("scale,expect", [(-130, fmdq.BASE_MIN), (110, fmdq.BASE_MAX)])
def test_base_is_clamped_to_the_accepted_range(scale, expect):
    d = wl.make_custom(32, 8, 8, 32, seed=14)
    delta = (d["x_t"].astype(np.float64) - d["x_prev"].astype(np.float64))
    x_p = np.zeros_like(d["x_prev"])
    x_t = (delta * 2.0 ** scale).astype(np.float32)
    assert np.isfinite(x_t).all() and (x_t != 0).any()
    assert fmdq.dynamic_base(x_t, x_p, 32, 1.0) == np.float32(expect)
