"""Parity of the SAR attention kernels (through the C ABI) with the CPU oracle.

Every stage is compared bit for bit: the FMDQ-INT8 codes and PoTs of Q, the
int8 codes and scales of K and V, the P cache (codes and PoTs of every kept
block) and the float32 output O of the cached and the reused step (both sides
form O from the same exact integer sums with the same roundings).  Inputs come
from the seeded generator ``gen/attention.py``; every device buffer starts as
garbage.
"""
import sys

import numpy as np
import pytest

from gen import attention as ga
from oracle import sar

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_mixed_precision_amd as dm
    dm.load()
    return dm


def run_gpu(dm, d, mask=None, reuse_v=None):
    """Cached step (and optionally one reused step) on cuda:0; returns numpy copies."""
    import torch
    dev = torch.device("cuda:0")
    B, H, L, dd = d["batch"], d["heads"], d["L"], d["d"]
    mask = d["mask"] if mask is None else mask
    att = dm.SarAttention(mask, B, H, L, dd, float(d["base_q"]), float(d["base_p"]), float(d["sm_scale"]), dev)
    for t, v in ((att.qcodes, 91), (att.qpot, 0xEE), (att.kcodes, 92), (att.vcodes_t, 93), (att.pcodes, 94),
                 (att.ppot, 0xDD)):
        t.fill_(v)
    att.kscale.fill_(float("nan"))
    att.out.fill_(float("nan"))
    q = torch.from_numpy(d["q"]).to(dev)
    k = torch.from_numpy(d["k"]).to(dev)
    v = torch.from_numpy(d["v"]).to(dev)
    log(f"  gpu cached step B={B} H={H} L={L} d={dd} nnz={att.nnz}")
    att.cached_step(q, k, v)
    torch.cuda.synchronize()
    res = dict(qcodes=att.qcodes.cpu().numpy(), qpot=att.qpot.cpu().numpy(), kcodes=att.kcodes.cpu().numpy(),
               kscale=att.kscale.cpu().numpy(), vcodes_t=att.vcodes_t.cpu().numpy(),
               vscale=att.vscale.cpu().numpy(), pcodes=att.pcodes.cpu().numpy()[:, :att.nnz],
               ppot=att.ppot.cpu().numpy()[:, :att.nnz], o=att.out.cpu().numpy().copy())
    if reuse_v is not None:
        log("  gpu reused step")
        att.reused_step(torch.from_numpy(reuse_v).to(dev))
        torch.cuda.synchronize()
        res["o_reused"] = att.out.cpu().numpy().copy()
        res["vscale_reused"] = att.vscale.cpu().numpy()
    return res


def compare(g, r, d):
    dd = d["d"]
    dp = g["qcodes"].shape[2]
    np.testing.assert_array_equal(g["qcodes"][:, :, :dd], r["qcodes"])
    assert (g["qcodes"][:, :, dd:] == 0).all()
    np.testing.assert_array_equal(g["qpot"][:, :, :dd], r["qpot"])
    assert (g["qpot"][:, :, dd:] == 0).all()
    np.testing.assert_array_equal(g["kcodes"][:, :, :dd], r["kcodes"])
    assert (g["kcodes"][:, :, dd:] == 0).all()
    np.testing.assert_array_equal(g["kscale"], r["kscale"])
    vct = g["vcodes_t"]
    np.testing.assert_array_equal(vct[:, :dd, :].transpose(0, 2, 1), r["vcodes"])
    assert (vct[:, dd:dp, :] == 0).all()
    np.testing.assert_array_equal(g["vscale"], r["vscale"])
    np.testing.assert_array_equal(g["ppot"], r["ppot"])
    np.testing.assert_array_equal(g["pcodes"], r["pcodes"])
    np.testing.assert_array_equal(g["o"], r["o"])


CASES = [
    # (batch, heads, L, d, density, seed)
    (1, 2, 256, 72, 0.63, 1),
    (2, 3, 512, 72, 0.5, 2),
    (1, 2, 256, 64, 0.63, 3),
    (1, 1, 256, 128, 0.63, 4),
    (1, 2, 192, 40, 0.8, 5),
    (1, 1, 64, 1, 1.0, 6),
    (2, 1, 128, 96, 1.0, 7),
    # more (head, query block) pairs than the scores kernel orders longest
    # first (1040 > 1024): its waves keep index order
    (1, 65, 1024, 16, 0.4, 18),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}L{c[2]}d{c[3]}" for c in CASES])
def test_sar_cached_and_reused_step_match_oracle(dm, case):
    B, H, L, dd, dens, seed = case
    d = ga.make_attention(B, H, L, dd, dens, seed)
    log(f"case B={B} H={H} L={L} d={dd} density={dens} seed={seed}")
    g = run_gpu(dm, d, reuse_v=d["v_next"])
    row_ptr, cols = sar.mask_to_csr(d["mask"])
    r = sar.cached_step(d["q"], d["k"], d["v"], row_ptr, cols, H, d["base_q"], d["sm_scale"], d["base_p"])
    compare(g, r, d)
    u = sar.reused_step(r["pcodes"], r["ppot"], d["v_next"], row_ptr, cols, H, d["base_p"])
    np.testing.assert_array_equal(g["vscale_reused"], u["vscale"])
    np.testing.assert_array_equal(g["o_reused"], u["o"])


PLANE_CASES = [
    # (d, q_outlier, log2 base_p, seed): outliers in Q raise its PoTs past 8
    # (more than two digit planes of a_Q); a small base_p raises P's PoTs past
    # 16 (four planes of a_P), a large one keeps them at or below 8 (two)
    (72, 2000.0, -15, 11),
    (128, 300.0, -28, 12),
    (72, 1.0, -28, 13),
    (40, 1.0, -4, 14),
    (1, 5000.0, -30, 15),
    (96, 1.0, -6, 16),
]


@pytest.mark.parametrize("case", PLANE_CASES, ids=[f"d{c[0]}q{c[1]:g}p{c[2]}" for c in PLANE_CASES])
def test_sar_digit_plane_counts_match_oracle(dm, case):
    """Every digit-plane count of a_Q (scores) and a_P (P·V), at several head
    widths: bit-equal to the oracle in every stage."""
    dd, qo, lbp, seed = case
    d = ga.make_attention(1, 2, 256, dd, 0.63, seed)
    rng = np.random.default_rng(seed)
    if qo != 1.0:
        hot = rng.random(d["q"].shape) < 0.002
        hot[0, 37, 0] = True
        d["q"] = np.where(hot, d["q"] * np.float32(qo), d["q"]).astype(np.float32)
    d["base_p"] = np.float32(2.0 ** lbp)
    log(f"case d={dd} q_outlier={qo} base_p=2^{lbp} seed={seed}")
    g = run_gpu(dm, d, reuse_v=d["v_next"])
    row_ptr, cols = sar.mask_to_csr(d["mask"])
    r = sar.cached_step(d["q"], d["k"], d["v"], row_ptr, cols, 2, d["base_q"], d["sm_scale"], d["base_p"])
    if qo != 1.0:
        assert r["qpot"].max() > 8
    compare(g, r, d)
    u = sar.reused_step(r["pcodes"], r["ppot"], d["v_next"], row_ptr, cols, 2, d["base_p"])
    np.testing.assert_array_equal(g["o_reused"], u["o"])


WIDE_CASES = [
    # (key outlier factor, Q outlier factor, seed): whole key rows scaled by
    # the factor spread a tile's logits far past 2^14, the range in which the
    # exponential needs no clamp at its cut-off; at 1e14, z − max z reaches
    # beyond 2^45, where the reduction of an unclamped argument loses its
    # leading bits and the polynomial overflows
    (2e4, 1.0, 21),
    (1e14, 1.0, 22),
    (1e14, 2000.0, 23),
]


def logit_spread(d, H):
    """Largest max − min of q·k·sm_scale (float64) over the kept keys of any
    32-row query tile."""
    L = d["L"]
    nb = L // 64
    best = 0.0
    for h in range(H):
        z = d["q"][h].astype(np.float64) @ d["k"][h].astype(np.float64).T * float(d["sm_scale"])
        for qb in range(nb):
            keys = np.concatenate([np.arange(kb * 64, kb * 64 + 64) for kb in np.nonzero(d["mask"][h, qb])[0]])
            for t in range(2):
                zz = z[qb * 64 + 32 * t:qb * 64 + 32 * t + 32][:, keys]
                best = max(best, float(zz.max() - zz.min()))
    return best


@pytest.mark.parametrize("case", WIDE_CASES, ids=[f"k{c[0]:g}q{c[1]:g}" for c in WIDE_CASES])
def test_sar_wide_logit_spread_matches_oracle(dm, case):
    """Tiles whose logits span more than 2^14 take the exponential with the
    clamp at its cut-off (E = 0 below it), up to spreads of 10^16 and more:
    bit-equal to the oracle in every stage, cached and reused step."""
    ko, qo, seed = case
    d = ga.make_attention(1, 2, 256, 72, 0.63, seed)
    rng = np.random.default_rng(seed)
    hot = rng.random(d["k"].shape[:2]) < 0.02
    d["k"] = np.where(hot[..., None], d["k"] * np.float32(ko), d["k"]).astype(np.float32)
    if qo != 1.0:
        hq = rng.random(d["q"].shape) < 0.002
        d["q"] = np.where(hq, d["q"] * np.float32(qo), d["q"]).astype(np.float32)
    spread = logit_spread(d, 2)
    log(f"case k_outlier={ko:g} q_outlier={qo:g} seed={seed} spread={spread:.3g}")
    assert spread > (1e5 if ko < 1e10 else 2.0 ** 46)
    g = run_gpu(dm, d, reuse_v=d["v_next"])
    row_ptr, cols = sar.mask_to_csr(d["mask"])
    r = sar.cached_step(d["q"], d["k"], d["v"], row_ptr, cols, 2, d["base_q"], d["sm_scale"], d["base_p"])
    if qo != 1.0:
        assert r["qpot"].max() > 8
    compare(g, r, d)
    u = sar.reused_step(r["pcodes"], r["ppot"], d["v_next"], row_ptr, cols, 2, d["base_p"])
    np.testing.assert_array_equal(g["o_reused"], u["o"])


def test_sar_empty_query_blocks_and_sparse_rows(dm):
    """Query blocks without any kept key block get O = 0; single kept blocks
    far from the diagonal work."""
    d = ga.make_attention(1, 2, 512, 72, 0.4, seed=8)
    mask = d["mask"].copy()
    mask[0, 3, :] = False
    mask[1, 7, :] = False
    mask[1, 0, :] = False
    mask[1, 0, 6] = True
    g = run_gpu(dm, d, mask=mask)
    row_ptr, cols = sar.mask_to_csr(mask)
    r = sar.cached_step(d["q"], d["k"], d["v"], row_ptr, cols, 2, d["base_q"], d["sm_scale"], d["base_p"])
    compare(g, r, d)
    assert (g["o"][0, 192:256] == 0).all() and (g["o"][1, 448:512] == 0).all()


def test_sar_closed_forms_on_gpu(dm):
    """Uniform attention (Q = 0, kept counts powers of two): P codes 64 at
    PoT 15 − log2 n and O the mean of the quantized V rows; bit-equal to the
    oracle as well."""
    import math
    L, dd, H = 512, 40, 2
    nb = L // 64
    rng = np.random.default_rng(6)
    mask = np.zeros((H, nb, nb), dtype=bool)
    for h in range(H):
        for qb in range(nb):
            mask[h, qb, rng.choice(nb, [1, 2, 4][(qb + h) % 3], replace=False)] = True
    d = ga.make_attention(1, H, L, dd, 0.5, seed=9)
    d["q"] = np.zeros_like(d["q"])
    g = run_gpu(dm, d, mask=mask)
    row_ptr, cols = sar.mask_to_csr(mask)
    assert (g["pcodes"] == 64).all()
    vc, vs = sar.quantize_v(d["v"])
    for h in range(H):
        for qb in range(nb):
            kbs = np.nonzero(mask[h, qb])[0]
            n = 64 * len(kbs)
            j0 = row_ptr[h * nb + qb]
            assert (g["ppot"][0, j0:j0 + len(kbs)] == 15 - int(math.log2(n))).all()
            keys = np.concatenate([np.arange(kb * 64, kb * 64 + 64) for kb in kbs])
            ref = (vc[h, keys].sum(axis=0).astype(np.float64) * vs[h].astype(np.float64) / n).astype(np.float32)
            assert (g["o"][h, qb * 64:(qb + 1) * 64] == ref[None, :]).all()


@pytest.mark.slow
def test_sar_full_size_sampled_heads(dm):
    """PixArt-α 1024 px attention (2 images × 16 heads, 4096 tokens, 72
    channels, 37% of the blocks pruned), in the launch configuration the
    benchmark times: the GPU runs every (image, head) pair; the oracle checks
    three of them completely (all stages, cached and reused step)."""
    spec = ga.ATTN_CONFIGS["pixart-alpha-1024px-attn"]
    d = ga.make_config("pixart-alpha-1024px-attn", seed=1)
    H = spec["heads"]
    g = run_gpu(dm, d, reuse_v=d["v_next"])
    row_ptr_all, cols_all = sar.mask_to_csr(d["mask"])
    nb = spec["L"] // 64
    for bh in (0, 17, 31):
        b, h = divmod(bh, H)
        log(f"  oracle (image {b}, head {h})")
        m1 = d["mask"][h:h + 1]
        row_ptr, cols = sar.mask_to_csr(m1)
        sl = slice(bh, bh + 1)
        r = sar.cached_step(d["q"][sl], d["k"][sl], d["v"][sl], row_ptr, cols, 1, d["base_q"], d["sm_scale"],
                            d["base_p"])
        u = sar.reused_step(r["pcodes"], r["ppot"], d["v_next"][sl], row_ptr, cols, 1, d["base_p"])
        dd = spec["d"]
        np.testing.assert_array_equal(g["qcodes"][sl, :, :dd], r["qcodes"])
        np.testing.assert_array_equal(g["qpot"][sl, :, :dd], r["qpot"])
        np.testing.assert_array_equal(g["kcodes"][sl, :, :dd], r["kcodes"])
        np.testing.assert_array_equal(g["kscale"][sl], r["kscale"])
        np.testing.assert_array_equal(g["vcodes_t"][sl, :dd].transpose(0, 2, 1), r["vcodes"])
        j0, j1 = row_ptr_all[h * nb], row_ptr_all[(h + 1) * nb]
        np.testing.assert_array_equal(g["pcodes"][b, j0:j1], r["pcodes"][0])
        np.testing.assert_array_equal(g["ppot"][b, j0:j1], r["ppot"][0])
        np.testing.assert_array_equal(g["o"][sl], r["o"])
        np.testing.assert_array_equal(g["o_reused"][sl], u["o"])


def test_sar_out_of_range_columns_are_ignored(dm):
    """Compressed-row entries outside [0, L/64) are skipped, as the header
    says: O, and the cache of every valid block, equal the oracle's on the mask
    without them; the cache entries of the skipped blocks are not written."""
    import torch
    dev = torch.device("cuda:0")
    B, H, L, dd = 1, 2, 256, 72
    nb = L // 64
    d = ga.make_attention(B, H, L, dd, 0.63, seed=17)
    row_ptr, cols = sar.mask_to_csr(d["mask"])
    rows = [list(cols[row_ptr[r]:row_ptr[r + 1]]) for r in range(H * nb)]
    rows[1] = [-1] + rows[1]                 # before the first kept block
    rows[5] = rows[5] + [nb + 3]             # after the last one
    rows[7] = rows[7] + [1000, 1 << 30]
    new_ptr = np.zeros(H * nb + 1, dtype=np.int32)
    new_ptr[1:] = np.cumsum([len(r) for r in rows])
    new_cols = np.array([c for r in rows for c in r], dtype=np.int32)
    valid = (new_cols >= 0) & (new_cols < nb)
    assert (~valid).sum() == 4 and valid.sum() == len(cols)
    nnz = len(new_cols)
    dp = dm.sar_padded_dim(dd)
    p = dm._binding.make_sar_params(B, H, L, dd, float(d["base_q"]), float(d["base_p"]), float(d["sm_scale"]))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, k, v, vn = t(d["q"]), t(d["k"]), t(d["v"]), t(d["v_next"])
    qc = torch.empty((B * H, L, dp), dtype=torch.int8, device=dev)
    qp = torch.empty((B * H, L // 32, dp), dtype=torch.uint8, device=dev)
    kc = torch.empty((B * H, L, dp), dtype=torch.int8, device=dev)
    ks = torch.empty((B * H, L), dtype=torch.float32, device=dev)
    vc = torch.empty((B * H, dp, L), dtype=torch.int8, device=dev)
    vs = torch.empty((B * H, dd), dtype=torch.float32, device=dev)
    pc = torch.full((B, nnz, 64, 64), 93, dtype=torch.int8, device=dev)
    pp = torch.full((B, nnz, 2, 64), 0xAB, dtype=torch.uint8, device=dev)
    out = torch.full((B * H, L, dd), float("nan"), dtype=torch.float32, device=dev)
    rp, cl = t(new_ptr), t(new_cols)
    log(f"  gpu cached step with {nnz - len(cols)} out-of-range column entries")
    dm.sar_quantize_q(p, q, qc, qp)
    dm.sar_quantize_k(p, k, kc, ks)
    dm.sar_quantize_v(p, v, vc, vs)
    dm.sar_scores(p, rp, cl, nnz, qc, qp, kc, ks, pc, pp)
    dm.sar_pv(p, rp, cl, nnz, pc, pp, vc, vs, out)
    torch.cuda.synchronize()
    g_out, g_pc, g_pp = out.cpu().numpy().copy(), pc.cpu().numpy(), pp.cpu().numpy()
    dm.sar_quantize_v(p, vn, vc, vs)
    dm.sar_pv(p, rp, cl, nnz, pc, pp, vc, vs, out)
    torch.cuda.synchronize()
    g_reused = out.cpu().numpy()
    r = sar.cached_step(d["q"], d["k"], d["v"], row_ptr, cols, H, d["base_q"], d["sm_scale"], d["base_p"])
    u = sar.reused_step(r["pcodes"], r["ppot"], d["v_next"], row_ptr, cols, H, d["base_p"])
    np.testing.assert_array_equal(g_out, r["o"])
    np.testing.assert_array_equal(g_reused, u["o"])
    np.testing.assert_array_equal(g_pc[:, valid], r["pcodes"])
    np.testing.assert_array_equal(g_pp[:, valid], r["ppot"])
    assert (g_pc[:, ~valid] == 93).all() and (g_pp[:, ~valid] == 0xAB).all()
