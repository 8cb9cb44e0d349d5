"""Pins of the oracle's 2-bit slice decomposition and slice stream (DSTAR §3.1
❷ ❸ ❹): the page's worked example (tests/golden/), exhaustive recomposition
of every code, the stream's order and shift encoding, and decoding the stream
by Horner accumulation against S computed by brute force in Python integers.
"""
import json
import os

import numpy as np
import pytest

from gen import workloads as wl
from oracle import fmdq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dstar_examples.json")
with open(GOLDEN) as f:
    EX = json.load(f)


def tags_for(tag, bits):
    return np.uint8(tag | ((bits // 2 - 1) << fmdq.PREC_SHIFT))


def test_slice_example_section_3_1():
    """70 -> slices 1, 0, 1, 2 (Slice[3] .. Slice[0]) at FPoT 1, 3, 5, 7, the
    first shift 2 (DSTAR §3.1 ❷, Fig. 5)."""
    ex = EX["slice_example"]
    sl = fmdq.code_slices(np.array([ex["value"]]), np.array([8]))
    assert [int(s[0]) for s in sl[::-1]] == ex["slices_hi_to_lo"]
    # one 8-bit sub-channel whose FPoT is 7 in the page's numbering: in tag
    # numbering the slices sit at tag, tag - 2, tag - 4, tag - 6
    g = 13
    codes = np.zeros((1, 1, 32), dtype=np.int64)
    codes[0, 0, 0] = ex["value"]
    ent, data, off = fmdq.slice_encode(codes, np.array([[tags_for(g, 8)]]))
    ns = [(int(e) >> 16) & 3 for e in ent[0, :4]]
    shifts = [int(e) >> 24 for e in ent[0, :4]]
    assert ns == [3, 2, 1, 0]                      # ascending FPoT: Slice[3] first
    fp = [ex["fpot_hi_to_lo"][0] + sum(shifts[1:i + 1]) for i in range(4)]
    assert fp == ex["fpot_hi_to_lo"] and shifts[1] == ex["first_shift"]
    assert [int(d[0]) & 3 for d in data[0, :4]] == [1, 0, 1, 2]
    assert off[0, -1] == 4


@pytest.mark.parametrize("bits", [2, 4, 6, 8])
def test_every_code_recomposes_from_its_slices(bits):
    pc = fmdq.PCEIL[bits]
    q = np.arange(-pc, pc + 1)
    sl = fmdq.code_slices(q, np.full(q.shape, bits))
    n = bits // 2
    rec = sum(sl[i] * 4 ** i for i in range(n))
    np.testing.assert_array_equal(rec, q)
    for i in range(n - 1):
        assert sl[i].min() >= 0 and sl[i].max() <= 3
    assert sl[n - 1].min() >= -2 and sl[n - 1].max() <= 1
    for i in range(n, 4):
        assert not sl[i].any()


@pytest.mark.parametrize("seed,rows,K,N,T,heavy", [(1, 96, 40, 12, 32, 0.1), (2, 70, 33, 8, 32, 0.3),
                                                   (3, 128, 24, 10, 64, 0.5), (4, 40, 17, 6, 16, 0.2)])
def test_stream_order_shifts_and_horner_decode(seed, rows, K, N, T, heavy):
    d = wl.make_custom(rows, K, N, T, seed=seed, heavy=heavy, c_range=(0.05, 500.0))
    codes, tags, _ = fmdq.quantize(d["x_t"], d["x_prev"], T, d["base"], d["k0"])
    ent, data, off = fmdq.slice_encode(codes, tags)
    w = d["w"].astype(np.int64)
    tg = fmdq.tag_of(tags)
    bits = fmdq.bits_of(tags)
    for tau in range(codes.shape[0]):
        E = int(off[tau, -1])
        assert E == int((bits[tau] // 2).sum())
        e = ent[tau, :E].astype(np.int64)
        k, n, sh = e & 0xFFFF, (e >> 16) & 3, e >> 24
        b = tg[tau][k] - 2 * n + fmdq.SLICE_TAG_OFF
        assert (np.diff(b) >= 0).all()
        same = np.diff(b) == 0
        assert (np.diff(k)[same] > 0).all()                    # ties by channel
        np.testing.assert_array_equal(sh[1:], np.diff(b))      # shift = FPoT step
        assert sh[0] == 0
        for beta in range(fmdq.SLICE_BINS + 1):
            assert off[tau, beta] == int((b < beta).sum())
        # Horner decode: acc <<= shift; acc += slice · W[k]; S = acc · 2^(15 - last tag)
        acc = np.zeros((T, N), dtype=object)
        for j in range(E):
            f = (data[tau, j][:, None] >> (2 * np.arange(4))) & 3
            f = f.reshape(-1).astype(np.int64)
            top = n[j] == bits[tau][k[j]] // 2 - 1
            v = np.where(top & (f >= 2), f - 4, f)
            acc = acc * (1 << int(sh[j])) + np.outer(v, w[k[j]]).astype(object)
        last = int(b[-1]) - fmdq.SLICE_TAG_OFF
        # brute force in Python integers: S = Σ_k q · 2^(15 - tag) · W[k]
        ref = np.zeros((T, N), dtype=object)
        for kk in range(K):
            ref = ref + np.outer(codes[tau, kk].astype(np.int64), w[kk]).astype(object) * (2 ** (15 - int(tg[tau, kk])))
        assert ((acc * (2 ** (15 - last))) == ref).all()
        assert (ent[tau, E:] == 0xFFFFFFFF).all()
