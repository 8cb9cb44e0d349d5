"""Pins of the oracle's GELU and MLP step.

GELU (tanh form, DSTAR §4.2/§4.3 fuse it into the linear; the reading is in the
oracle) is checked against torch's own tanh-approximate GELU evaluated in
float64, against the tanh formula and the exact identity GELU(x) − GELU(−x) = x,
and at its limits.  The MLP step is checked against two separate layer calls
with an independently computed GELU in between.
"""
import math

import numpy as np
import pytest
import torch

from gen import workloads as wl
from oracle import fmdq


def assert_close_to_tanh_form(got, ref, y):
    """float32 rounding of the value (2^-23 relative) plus the float64
    cancellation of 1 + tanh(u) in the reference formula at negative y
    (absolute error up to a few ulp of |y| in float64)."""
    got = np.asarray(got, dtype=np.float64)
    bound = 2.0 ** -23 * np.abs(ref) + 2.0 ** -50 * np.abs(np.asarray(y, dtype=np.float64)) + 1e-40
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (np.asarray(y)[bad][:5], got[bad][:5], np.asarray(ref)[bad][:5])


def test_gelu_matches_torch_tanh_gelu_in_float64():
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.standard_normal(20000) * 3, rng.uniform(-12, 12, 5000)]).astype(np.float32)
    ref = torch.nn.functional.gelu(torch.from_numpy(y.astype(np.float64)), approximate="tanh").numpy()
    # the same function in float64; the oracle rounds once to float32
    assert_close_to_tanh_form(fmdq.gelu(y), ref, y)


def test_gelu_tanh_formula_and_odd_part_identity():
    y = np.linspace(-6, 6, 2001).astype(np.float32)
    y64 = y.astype(np.float64)
    tanh_form = 0.5 * y64 * (1 + np.tanh(math.sqrt(2 / math.pi) * (y64 + 0.044715 * y64 ** 3)))
    assert_close_to_tanh_form(fmdq.gelu(y), tanh_form, y)
    # GELU(x) - GELU(-x) = x for the tanh form (0.5x(1+t) + 0.5x(1-t))
    d = fmdq.gelu(y).astype(np.float64) - fmdq.gelu(-y).astype(np.float64)
    np.testing.assert_allclose(d, y64, rtol=2 ** -21, atol=2 ** -24)


def test_gelu_limits():
    assert fmdq.gelu(np.float32([0.0]))[0] == 0.0
    assert fmdq.gelu(np.float32([30.0]))[0] == np.float32(30.0)       # saturates to y
    assert fmdq.gelu(np.float32([-30.0]))[0] == 0.0                    # underflows to 0
    big = fmdq.gelu(np.float32([1e30, -1e30]))
    assert big[0] == np.float32(1e30) and big[1] == 0.0
    tiny = fmdq.gelu(np.float32([1e-20]))[0]                          # ≈ y/2 near 0
    assert tiny == np.float32(0.5e-20)


def test_mlp_step_is_two_layers_with_gelu_between():
    d1 = wl.make_custom(70, 48, 96, 32, seed=51)
    d2 = wl.make_custom(70, 96, 48, 32, seed=52)
    y1p = d1["y_prev"]
    gp = fmdq.gelu(y1p)
    fc1 = dict(w=d1["w"], w_scale=d1["w_scale"], base=d1["base"])
    fc2 = dict(w=d2["w"], w_scale=d2["w_scale"], base=np.float32(0.01))
    y1, g, y2, h1, h2 = fmdq.mlp_step(d1["x_t"], d1["x_prev"], y1p, gp, d2["y_prev"], fc1, fc2, 32, 2)
    r1 = fmdq.layer(d1["x_t"], d1["x_prev"], d1["w"], d1["w_scale"], y1p, d1["base"], 32, 2)
    np.testing.assert_array_equal(y1, r1["y"])
    g_ref = torch.nn.functional.gelu(torch.from_numpy(r1["y"].astype(np.float64)), approximate="tanh")
    assert_close_to_tanh_form(g, g_ref.numpy(), r1["y"])
    r2 = fmdq.layer(g, gp, d2["w"], d2["w_scale"], d2["y_prev"], np.float32(0.01), 32, 2)
    np.testing.assert_array_equal(y2, r2["y"])
    assert h1.sum() == 3 * 48 and h2.sum() == 3 * 96
