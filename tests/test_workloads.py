"""The input generators: the walk drawn at once equals the per-pair draws."""
import numpy as np

from gen import workloads as wl


def test_walk_matches_per_pair_inputs():
    xs = wl.make_walk(0, "fc1", 1)
    d = wl.make_inputs(0, "fc1", 1)
    np.testing.assert_array_equal(xs[0], d["x_prev"])
    np.testing.assert_array_equal(xs[1], d["x_t"])


def test_profiled_base_is_half_the_median_channel_rms():
    rng = np.random.default_rng(0)
    sig = np.array([0.5, 1.0, 2.0, 4.0, 8.0])
    d = rng.standard_normal((20000, 5)) * sig
    b = wl.profiled_base(d)
    assert abs(float(b) - 1.0) < 0.02 and b.dtype == np.float32
