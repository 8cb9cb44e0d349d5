"""Property tests of the oracle over random shapes and value scales (CPU).

Hypothesis draws the shape (ragged last tiles included), the token tile, k0,
the base and, per input channel, the scale of Δ: exact zeros, float32
subnormals, ordinary values, and values far above base·2^21 that saturate the
PoT.  Each case is checked against definitions written element by element:
the PoT as the smallest j with M ≤ base·2^j (DSTAR §3.1 Eq. 3, closed upper
edges, capped at 21), codes within ±PCeil and within half a step where
unsaturated, the codes and Y of an exact-rational brute-force layer, and the
bucket as a stable order by (FPoT tag ascending, precision descending).
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import fmdq
from test_oracle_pins import _brute_force_layer

SCALES = [0.0, 1e-41, 1e-3, 1.0, 30.0, 1e30]


@st.composite
def layers(draw):
    T = draw(st.sampled_from([16, 32, 64]))
    rows = draw(st.integers(1, 2 * T + 7))
    K = draw(st.integers(1, 12))
    N = draw(st.integers(1, 4))
    k0 = draw(st.integers(1, 15))
    base = float(np.float32(2.0 ** draw(st.integers(-20, 10)) * draw(st.floats(1.0, 1.99))))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    scales = draw(st.lists(st.sampled_from(SCALES), min_size=K, max_size=K))
    rng = np.random.default_rng(seed)
    x_prev = (rng.standard_normal((rows, K)) * rng.choice([0.0, 1.0, 100.0], K)).astype(np.float32)
    delta = rng.standard_normal((rows, K)) * np.array(scales)[None, :]
    x_t = (x_prev.astype(np.float64) + delta).astype(np.float32)
    if draw(st.booleans()):            # a subnormal difference with x_prev = 0
        x_prev[:, 0] = 0.0
        x_t[:, 0] = np.float32(1e-42) * rng.integers(-3, 4, rows).astype(np.float32)
    return dict(x_t=x_t, x_prev=x_prev, w=rng.integers(-127, 128, (K, N)).astype(np.int8),
                w_scale=rng.uniform(1e-3, 1e-2, N).astype(np.float32),
                y_prev=rng.standard_normal((rows, N)).astype(np.float32),
                base=np.float32(base), token_tile=T, k0=k0)


SETTINGS = settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@SETTINGS
@given(layers())
def test_pot_codes_and_bucket_follow_their_definitions(d):
    T, k0 = d["token_tile"], d["k0"]
    rows, K = d["x_t"].shape
    b = float(np.float32(d["base"]))
    codes, tags, hist = fmdq.quantize(d["x_t"], d["x_prev"], T, d["base"], k0)
    perm, off = fmdq.bucket(tags)
    tag, bits = fmdq.tag_of(tags), fmdq.bits_of(tags)
    e = fmdq.step_exponent(tag)
    nt = codes.shape[0]
    assert hist.sum() == nt * K
    for tau in range(nt):
        r0, r1 = tau * T, min(rows, tau * T + T)
        for k in range(K):
            dl = (d["x_t"][r0:r1, k] - d["x_prev"][r0:r1, k]).astype(np.float32).astype(np.float64)
            m = float(np.abs(dl).max())
            pot = next((j for j in range(22) if m <= b * 2.0 ** j), 21)   # exact: b·2^j is a float
            bt = 2 if pot <= k0 else 4 if pot <= k0 + 2 else 6 if pot <= k0 + 4 else 8
            assert int(bits[tau, k]) == bt
            assert int(e[tau, k]) == pot - (bt - 2)
            q = codes[tau, k, : r1 - r0].astype(np.int64)
            pc = 2 ** (bt - 2)
            assert np.abs(q).max() <= pc
            assert not codes[tau, k, r1 - r0:].any()
            step = b * 2.0 ** int(e[tau, k])
            if m <= b * 2.0 ** 21:                       # unsaturated: half a step
                assert (np.abs(dl - q * step) <= step * (0.5 + 2.0 ** -16)).all()
            else:                                        # saturated: the largest values clip
                assert np.abs(q).max() == pc
        # bucket: a permutation in (tag asc, precision desc, channel asc) order
        p = perm[tau].astype(np.int64)
        assert sorted(p.tolist()) == list(range(K))
        key = [(int(tag[tau, c]), -int(bits[tau, c]), c) for c in p]
        assert key == sorted(key)
        for g in range(16):
            assert off[tau][4 * g] == int((tag[tau] < g).sum())
        assert off[tau][-1] == K


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(layers())
def test_layer_matches_exact_rational_brute_force(d):
    T = d["token_tile"]
    r = fmdq.layer(d["x_t"], d["x_prev"], d["w"], d["w_scale"], d["y_prev"], d["base"], T, d["k0"])
    codes, y_bf, _ = _brute_force_layer(d)
    for (row, k), q in codes.items():
        assert r["codes"][row // T, k, row % T] == q
    ulp = np.spacing(np.abs(y_bf).astype(np.float32)).astype(np.float64)
    assert (np.abs(r["y"].astype(np.float64) - y_bf.astype(np.float64)) <= ulp).all()
