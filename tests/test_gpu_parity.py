"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer stages (codes, tags, bit histogram, bucket order, group offsets and the
int32 group accumulators) must match bit for bit; Y_t must satisfy
|y_gpu − y_oracle| ≤ 1e-5 · (|Y_{t−1}| + |Y_t − Y_{t−1}|) elementwise (the
float32 combine tolerance), and the number of bit-identical outputs is
reported.  Inputs come from the seeded generators in ``gen/``.
"""
import sys
import time

import numpy as np
import pytest

from gen import workloads as wl
from oracle import fmdq
from tests import digits

pytestmark = pytest.mark.gpu

REL_TOL = 1e-5


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


def gpu_layer(dm, d, dbg=None, inplace=False, y_prev_np=None, dynamic=False, sdump=None,
              plain_codes=True):
    """Runs the three stages on cuda:0; every output buffer starts as garbage.

    Stage 3 runs twice from the same codes: once as the product path (no
    accumulator dump: the MFMA kernel where the shape allows it) -> "y", with
    the exact S of the tiles in ``sdump`` (default: ``dbg``) dumped by that
    same kernel -> "s"; and, when ``dbg`` names a tile range, once more with
    the group accumulators dumped (the per-group kernel) -> "y_dbg" and
    "acc".  With ``dynamic`` the base is found on the device first
    (dynamic_base -> "base") and stages 1 and 3 read it from there
    (quantize_dyn, linear_dyn).  With ``plain_codes=False`` stages 1 and 3
    get no plain-codes buffer (stage 1 writes only tags, aligned codes and
    digit planes)."""
    import torch
    dev = torch.device("cuda:0")
    rows, K, N, T = d["rows"], d["K"], d["N"], d["token_tile"]
    nt = (rows + T - 1) // T
    x_t = torch.from_numpy(d["x_t"]).to(dev)
    x_p = torch.from_numpy(d["x_prev"]).to(dev)
    w = torch.from_numpy(d["w"]).to(dev)
    ws = torch.from_numpy(d["w_scale"]).to(dev)
    y_np = d["y_prev"] if y_prev_np is None else y_prev_np
    y0 = torch.from_numpy(y_np).to(dev)
    p = dm.make_params(rows, K, T, float(d["base"]), d["k0"], d["tokens_per_seq"])
    codes = torch.full((nt, K, T), 90, dtype=torch.int8, device=dev) if plain_codes else None
    tags = torch.full((nt, K), 0xEE, dtype=torch.uint8, device=dev)
    acodes = torch.full((nt * T, K), 77, dtype=torch.int8, device=dev)
    hcodes = torch.full((2, nt, K, T), 66, dtype=torch.int8, device=dev)
    w_t = torch.full((N, K), 55, dtype=torch.int8, device=dev)
    hist = torch.zeros(4, dtype=torch.int32, device=dev)
    perm = torch.full((nt, K), -1, dtype=torch.int16, device=dev)
    off = torch.full((nt, 65), -7, dtype=torch.int32, device=dev)
    y1 = y0 if inplace else torch.full((rows, N), float("nan"), dtype=torch.float32, device=dev)
    dm.pack_weights(K, N, w, w_t)
    base = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
    if dynamic:
        dm.dynamic_base(p, x_t, x_p, base)
        dm.quantize_dyn(p, base, x_t, x_p, codes, tags, acodes, hcodes, hist)
    else:
        dm.quantize(p, x_t, x_p, codes, tags, acodes, hcodes, hist)
    dm.bucket(p, tags, perm, off)
    sd = sdump if sdump is not None else dbg
    s_dbg, slo, shi = None, 0, 0
    if sd is not None:
        slo, shi = sd
        s_dbg = torch.full((shi - slo, T, N), 0x5A5A5A5A5A5A, dtype=torch.int64, device=dev)
    if dynamic:
        dm.linear_dyn(p, base, N, codes, perm, off, acodes, hcodes, w, w_t, ws, y0, y1,
                      dbg_tile_lo=slo, dbg_tile_hi=shi, s_dbg=s_dbg)
    else:
        dm.linear(p, N, codes, perm, off, acodes, hcodes, w, w_t, ws, y0, y1,
                  dbg_tile_lo=slo, dbg_tile_hi=shi, s_dbg=s_dbg)
    out = dict(codes=codes, tags=tags, acodes=acodes, hcodes=hcodes, w_t=w_t, hist=hist, perm=perm,
               group_off=off, y=y1, base=base)
    if s_dbg is not None:
        out["s"] = s_dbg
    if dbg is not None:
        lo, hi = dbg
        acc = torch.full((hi - lo, 16, T, N), 0x7777, dtype=torch.int32, device=dev)
        y0b = torch.from_numpy(y_np).to(dev)
        y2 = torch.full((rows, N), float("nan"), dtype=torch.float32, device=dev)
        if dynamic:
            dm.linear_dyn(p, base, N, codes, perm, off, acodes, hcodes, w, w_t, ws, y0b, y2, acc, lo, hi)
        else:
            dm.linear(p, N, codes, perm, off, acodes, hcodes, w, w_t, ws, y0b, y2, acc, lo, hi)
        out.update(acc=acc, y_dbg=y2)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in out.items() if v is not None}
    out["perm"] = out["perm"].view(np.uint16)
    return out


def par_linear(codes, tags, perm, off, w, w_scale, y_prev, base, T):
    """fmdq.linear over every token tile, run on chunks of tiles in parallel
    threads (one BLAS thread each): the oracle's own function, called per
    chunk; the rows of each chunk are taken from its call."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    rows = y_prev.shape[0]
    nt = (rows + T - 1) // T
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    chunks = [c for c in np.array_split(np.arange(nt), 2 * workers) if len(c)]
    y = np.array(y_prev, dtype=np.float32, copy=True)

    def run(ch):
        return ch, fmdq.linear(codes, tags, perm, off, w, w_scale, y_prev, base, T, tiles=ch)

    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        for ch, yy in ex.map(run, chunks):
            r0, r1 = int(ch[0]) * T, min((int(ch[-1]) + 1) * T, rows)
            y[r0:r1] = yy[r0:r1]
    return y


def check_y(y_gpu, y_orc, y_prev, what=""):
    y_gpu = y_gpu.astype(np.float64)
    y_orc = y_orc.astype(np.float64)
    y_prev = y_prev.astype(np.float64)
    assert np.isfinite(y_gpu).all(), f"{what}: non-finite output"
    den = np.abs(y_prev) + np.abs(y_orc - y_prev)
    err = np.abs(y_gpu - y_orc)
    rel = np.where(den > 0, err / np.where(den > 0, den, 1.0), np.where(err > 0, np.inf, 0.0))
    exact = int((y_gpu == y_orc).sum())
    log(f"  {what}: max rel err {rel.max():.3e}, bit-identical {exact}/{y_gpu.size}")
    assert rel.max() <= REL_TOL, f"{what}: max rel err {rel.max()}"
    # S is an exact integer on both sides and the float64 combine is the same
    # sequence of correctly rounded operations, so the outputs are identical.
    assert exact == y_gpu.size, f"{what}: {y_gpu.size - exact} outputs differ from the oracle"


def check_integer_stages(g, codes, tags, hist, perm, off, what="", w=None):
    np.testing.assert_array_equal(g["codes"], codes, err_msg=f"{what}: codes")
    np.testing.assert_array_equal(g["tags"], tags, err_msg=f"{what}: tags")
    # stage 3's 8-bit operands, by identity against the oracle's codes and tags
    digits.check_operands(g["acodes"], g["hcodes"], codes, tags, what)
    if w is not None:
        np.testing.assert_array_equal(g["w_t"], w.T, err_msg=f"{what}: packed weights")
    np.testing.assert_array_equal(g["hist"].astype(np.int64), hist, err_msg=f"{what}: bit histogram")
    np.testing.assert_array_equal(g["perm"], perm, err_msg=f"{what}: bucket order")
    np.testing.assert_array_equal(g["group_off"], off, err_msg=f"{what}: group offsets")


def full_compare(dm, d, inplace=False, dump=True):
    rows, T = d["rows"], d["token_tile"]
    nt = (rows + T - 1) // T
    log(f"case {d['name']} rows={rows} K={d['K']} N={d['N']} T={T} inplace={inplace}")
    g = gpu_layer(dm, d, dbg=(0, nt) if dump else None, inplace=inplace)
    codes, tags, hist = fmdq.quantize(d["x_t"], d["x_prev"], T, d["base"], d["k0"])
    perm, off = fmdq.bucket(tags)
    check_integer_stages(g, codes, tags, hist, perm, off, d["name"], d["w"])
    if not dump:
        y = fmdq.linear(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], d["base"], T)
        check_y(g["y"], y, d["y_prev"], d["name"])
        return g, y
    y, accs = fmdq.linear(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], d["base"], T,
                          return_acc=True)
    for tau in range(nt):
        np.testing.assert_array_equal(g["acc"][tau].astype(np.int64), accs[tau],
                                      err_msg=f"{d['name']}: group accumulators of tile {tau}")
    check_s(g["s"], accs, range(nt), 0, d["name"])
    y_prev = d["y_prev"]
    check_y(g["y_dbg"], y, y_prev, d["name"] + " (per-group kernel)")
    check_y(g["y"], y, y_prev, d["name"])
    return g, y


def check_s(s_gpu, accs, tiles, lo, what=""):
    """The product kernel's exact integer S of each tile against the oracle's
    per-FPoT-group accumulators aligned by shifts (shift_combine)."""
    for tau in tiles:
        np.testing.assert_array_equal(s_gpu[tau - lo], fmdq.shift_combine(accs[tau]),
                                      err_msg=f"{what}: S of tile {tau} (product kernel)")
    log(f"  {what}: S of {len(list(tiles))} tiles bit-exact (product kernel)")


SMALL = [
    dict(rows=96, K=64, N=64, T=32, seed=1),
    dict(rows=70, K=48, N=40, T=32, seed=2),                       # ragged last tile
    dict(rows=128, K=36, N=36, T=64, seed=3),
    dict(rows=40, K=33, N=20, T=16, seed=4),                       # odd K
    dict(rows=200, K=130, N=24, T=32, seed=5),                     # K % 4 == 2
    dict(rows=256, K=300, N=520, T=32, seed=6, heavy=0.3),
    dict(rows=160, K=96, N=132, T=32, seed=7, heavy=0.5, c_range=(0.01, 3000.0)),  # many groups
    dict(rows=128, K=64, N=48, T=32, seed=8, tokens_per_seq=64),   # batch of two sequences
    dict(rows=300, K=1152, N=256, T=64, seed=9),                   # ragged T=64
    dict(rows=33, K=2048, N=128, T=32, seed=10, heavy=0.1),        # one row in the last tile
    # every sub-channel heavy: most channels need their own FPoT groups
    dict(rows=96, K=4096, N=96, T=32, seed=21, heavy=1.0, c_range=(4.0, 8.0)),
    dict(rows=128, K=8192, N=64, T=64, seed=22, heavy=1.0, c_range=(4.0, 8.0)),
    # more such channels than the MFMA kernel stages: exact per-group fallback
    dict(rows=64, K=8192, N=72, T=32, seed=20, heavy=1.0, c_range=(4.0, 8.0)),
    dict(rows=200, K=1536, N=260, T=32, seed=23, heavy=0.2, c_range=(0.5, 64.0)),
    # channels with PoT >= 14 (third digits) through the MFMA kernel
    dict(rows=160, K=1152, N=132, T=32, seed=24, heavy=0.3, c_range=(0.02, 4000.0)),  # N % 16 != 0
    dict(rows=192, K=640, N=256, T=64, seed=25, heavy=0.3, c_range=(0.02, 4000.0)),
    dict(rows=128, K=1152, N=144, T=32, seed=26, heavy=0.15, c_range=(0.05, 2000.0)),
    # K % 64 != 0 (a multiple of 16): the product kernels' partial last chunk
    dict(rows=64, K=16, N=64, T=32, seed=27),
    dict(rows=300, K=1040, N=264, T=32, seed=28, heavy=0.2, c_range=(0.02, 4000.0)),
    dict(rows=256, K=1072, N=132, T=64, seed=29, heavy=0.3, c_range=(0.02, 4000.0)),
    # T = 16 through the MFMA kernel (two token tiles per 32-row block)
    dict(rows=200, K=1152, N=260, T=16, seed=36, heavy=0.3, c_range=(0.02, 4000.0)),  # d2, ragged
    dict(rows=96, K=4096, N=96, T=16, seed=37, heavy=1.0, c_range=(4.0, 8.0)),
    dict(rows=64, K=8192, N=72, T=16, seed=38, heavy=1.0, c_range=(4.0, 8.0)),
]

# Limits of the ABI: the largest K (the bucket's global-memory variant above
# K = 32768), the largest K that the MFMA kernel takes, the largest N, one row.
EDGE = [
    dict(rows=32, K=65535, N=16, T=32, seed=30),
    dict(rows=40, K=40000, N=20, T=16, seed=31, heavy=0.1),
    dict(rows=64, K=65472, N=32, T=32, seed=32, heavy=0.05),
    dict(rows=32, K=64, N=1 << 20, T=32, seed=33),
    dict(rows=1, K=64, N=64, T=32, seed=34),
    dict(rows=1, K=5, N=4, T=64, seed=35),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c['rows']}x{c['K']}x{c['N']}-T{c['T']}-s{c['seed']}")
def test_small_layers_match_oracle(dm, case):
    c = dict(case)
    d = wl.make_custom(c.pop("rows"), c.pop("K"), c.pop("N"), c.pop("T"), c.pop("seed"), **c)
    full_compare(dm, d)


@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"{c['rows']}x{c['K']}x{c['N']}-T{c['T']}-s{c['seed']}")
def test_abi_limits_match_oracle(dm, case):
    """(The group-accumulator dump is skipped at N = 2^20: it would be 2 GiB.)"""
    c = dict(case)
    d = wl.make_custom(c.pop("rows"), c.pop("K"), c.pop("N"), c.pop("T"), seed=c.pop("seed"), **c)
    full_compare(dm, d, dump=d["N"] <= 65536)


def aligned_workspace(torch, nbytes, dev):
    """A uint8 device tensor of nbytes whose data pointer is 256-byte aligned."""
    raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    off = (-raw.data_ptr()) % 256
    return raw[off:off + nbytes]


@pytest.mark.parametrize("case", [SMALL[0], SMALL[1], SMALL[3], SMALL[8], SMALL[13], SMALL[14]],
                         ids=lambda c: f"{c['rows']}x{c['K']}x{c['N']}-T{c['T']}-s{c['seed']}")
def test_one_call_layer_matches_oracle(dm, case):
    """dstar_fmdq_layer (the three stages in one call, intermediates in a
    caller workspace): Y_t bit for bit and the bit histogram, against the
    oracle; the workspace holds the codes and tags afterwards."""
    import torch
    dev = torch.device("cuda:0")
    c = dict(case)
    d = wl.make_custom(c.pop("rows"), c.pop("K"), c.pop("N"), c.pop("T"), seed=c.pop("seed"), **c)
    rows, K, N, T = d["rows"], d["K"], d["N"], d["token_tile"]
    log(f"case {d['name']} (one-call layer)")
    p = dm.make_params(rows, K, T, float(d["base"]), d["k0"], d["tokens_per_seq"])
    need = dm.layer_workspace_size(p)
    ws = aligned_workspace(torch, need, dev)
    ws.fill_(0xA5)
    w = torch.from_numpy(d["w"]).to(dev)
    w_t = torch.empty((N, K), dtype=torch.int8, device=dev)
    dm.pack_weights(K, N, w, w_t)
    y0 = torch.from_numpy(d["y_prev"]).to(dev)
    y1 = torch.full((rows, N), float("nan"), dtype=torch.float32, device=dev)
    hist = torch.zeros(4, dtype=torch.int32, device=dev)
    dm.layer(p, N, torch.from_numpy(d["x_t"]).to(dev), torch.from_numpy(d["x_prev"]).to(dev), w, w_t,
             torch.from_numpy(d["w_scale"]).to(dev), y0, y1, ws, hist)
    torch.cuda.synchronize()
    r = fmdq.layer(d["x_t"], d["x_prev"], d["w"], d["w_scale"], d["y_prev"], d["base"], T, d["k0"])
    check_y(y1.cpu().numpy(), r["y"], d["y_prev"], d["name"] + " (one call)")
    np.testing.assert_array_equal(hist.cpu().numpy().astype(np.int64), r["hist"])
    nt = (rows + T - 1) // T
    np.testing.assert_array_equal(ws[:nt * K * T].cpu().numpy().view(np.int8).reshape(nt, K, T), r["codes"])


def test_zero_delta_gives_cached_output_bit_exact(dm):
    d = wl.make_custom(96, 64, 40, 32, seed=12, zero_delta=True)
    g, y = full_compare(dm, d)
    np.testing.assert_array_equal(g["y"], d["y_prev"])


def test_in_place_update(dm):
    d = wl.make_custom(130, 80, 36, 32, seed=13, heavy=0.2)
    full_compare(dm, d, inplace=True)


def test_saturated_and_extreme_subchannels(dm):
    rng = np.random.default_rng(14)
    rows, K, N, T = 64, 40, 16, 32
    base = np.float32(0.01)
    x_prev = rng.standard_normal((rows, K)).astype(np.float32)
    delta = rng.standard_normal((rows, K)) * 0.01
    delta[3, 1] = base * 2.0 ** 23            # beyond base·2^21: PoT 21, clipped codes
    delta[40, 2] = -base * 2.0 ** 21          # exactly at the last bin edge
    delta[41, 3] = base * 2.0 ** 12
    delta[:, 5] = 0.0                          # all-zero sub-channels
    delta[7, 6] = base                         # exactly base: PoT 0
    x_t = (x_prev.astype(np.float64) + delta).astype(np.float32)
    d = dict(x_t=x_t, x_prev=x_prev, w=rng.integers(-127, 128, (K, N)).astype(np.int8),
             w_scale=rng.uniform(1e-3, 1e-2, N).astype(np.float32),
             y_prev=rng.standard_normal((rows, N)).astype(np.float32), base=base, k0=2,
             token_tile=T, rows=rows, tokens_per_seq=rows, K=K, N=N, name="extreme")
    for k0 in (1, 2, 6, 15):
        d["k0"] = k0
        d["name"] = f"extreme-k0={k0}"
        full_compare(dm, d)


def test_t16_block_with_one_ineligible_tile(dm):
    """T = 16: the two token tiles of the first 32-row block differ in
    eligibility (tile 1 has sixteen sub-channels at PoT 21, so 128·Σ 2^PoT
    reaches 2^31 and it takes the exact per-group path) while tile 0 and the
    next block's tiles (one with a third digit) go through the MFMA sums."""
    rng = np.random.default_rng(39)
    rows, K, N, T = 64, 64, 48, 16
    base = np.float32(0.01)
    x_prev = rng.standard_normal((rows, K)).astype(np.float32)
    delta = rng.standard_normal((rows, K)) * 0.05
    delta[16, :16] = base * 2.0 ** 21
    delta[40, 20] = -base * 2.0 ** 15
    delta[50, 21] = base * 2.0 ** 9
    x_t = (x_prev.astype(np.float64) + delta).astype(np.float32)
    d = dict(x_t=x_t, x_prev=x_prev, w=rng.integers(-128, 128, (K, N)).astype(np.int8),
             w_scale=rng.uniform(1e-3, 1e-2, N).astype(np.float32),
             y_prev=rng.standard_normal((rows, N)).astype(np.float32), base=base, k0=2,
             token_tile=T, rows=rows, tokens_per_seq=rows, K=K, N=N, name="t16-mixed")
    full_compare(dm, d)


def test_second_digit_dense_pass(dm):
    """A workgroup whose second-digit lists outnumber its dense chunks takes
    the masked dense pass over the second digits (32-row tiles, N % 16 == 0,
    K <= 8192): here with a ragged last tile, a partial last chunk
    (K % 64 = 16), an ineligible tile (sixteen sub-channels at PoT 21) and
    third digits in another; every integer stage, S and Y_t bit for bit."""
    rows, K, N, T = 120, 1040, 64, 32
    d = wl.make_custom(rows, K, N, T, seed=47, heavy=1.0, c_range=(4.0, 8.0))
    base = float(d["base"])
    x = d["x_prev"].astype(np.float64)
    d["x_t"][32, :16] = (x[32, :16] + base * 2.0 ** 21).astype(np.float32)      # tile 1 ineligible
    d["x_t"][70, 100:104] = (x[70, 100:104] - base * 2.0 ** 14.5).astype(np.float32)   # tile 2: PoT 15
    delta = fmdq.differential(d["x_t"], d["x_prev"])
    pot = fmdq.pot_exponent(fmdq.subchannel_max(delta, T), d["base"])
    elig = [128 * np.sum(2.0 ** pot[t].astype(np.int64)) < 2 ** 31 for t in range(4)]
    units = sum(int(np.ceil((pot[t] >= 7).sum() / 64)) for t in range(4) if elig[t])
    assert elig == [True, False, True, True] and units > (K + 63) // 64 and (pot[2] >= 14).sum() == 4
    full_compare(dm, d)


def test_config0_full(dm):
    d = wl.make_inputs(0, "fc1", 1)
    t = time.time()
    full_compare(dm, d)
    log(f"  config 0 done in {time.time() - t:.1f}s")


BUCKET_K = [1024, 1025, 2048, 2049, 4096, 4097, 8192, 8193, 12288, 16383, 16384, 16385]


@pytest.mark.parametrize("K", BUCKET_K)
def test_bucket_chunk_counts_match_oracle(dm, K):
    """Stage 2 alone on seeded tag bytes, at both sides of every boundary of
    its instantiations (1, 2, 4, 8 or 16 chunks of 64 channels per wave, and
    the other variant above K = 16384): perm and offsets bit-equal to the
    oracle.  Tiles: skewed over a few bins, uniform over all 64, and a single
    bin."""
    import torch
    dev = torch.device("cuda:0")
    T, nt = 32, 3
    rng = np.random.default_rng(K)
    g = np.minimum(rng.geometric(0.35, size=(nt, K)) - 1, 15)
    pc = rng.choice(4, size=(nt, K), p=[0.1, 0.2, 0.3, 0.4])
    g[1] = rng.integers(0, 16, size=K)
    pc[1] = rng.integers(0, 4, size=K)
    g[2], pc[2] = 7, 2
    tags = (g | (pc << fmdq.PREC_SHIFT)).astype(np.uint8)
    perm_r, off_r = fmdq.bucket(tags)
    p = dm.make_params(nt * T, K, T, 1.0, 2, nt * T)
    tg = torch.from_numpy(tags).to(dev)
    perm = torch.full((nt, K), -1, dtype=torch.int16, device=dev)
    off = torch.full((nt, 65), -7, dtype=torch.int32, device=dev)
    log(f"  gpu bucket K={K}")
    dm.bucket(p, tg, perm, off)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(perm.cpu().numpy().view(np.uint16), perm_r)
    np.testing.assert_array_equal(off.cpu().numpy(), off_r)


def test_determinism(dm):
    """Ten runs of the same layer give the same bits in every output (the
    stages have no atomics whose order could change a result)."""
    d = wl.make_custom(512, 1152, 640, 32, seed=15, heavy=0.05)
    a = gpu_layer(dm, d, dbg=(0, 16))
    for r in range(9):
        b = gpu_layer(dm, d, dbg=(0, 16))
        for k in a:
            np.testing.assert_array_equal(a[k], b[k], err_msg=f"run {r + 2}: {k}")
    log("  10 runs bit-identical")


def w_minus_128_case(K, T, pot_heavy, n_heavy, seed):
    """One token tile at the int32 exactness bound of the product kernel:
    n_heavy channels whose Δ is −base·2^pot_heavy in every row (code −64 at
    step 2^(pot_heavy−6), a = −2^pot_heavy), the other channels small, and W
    = −128 on the heavy channels of column 0 (|S| reaches 128·Σ 2^PoT there).
    """
    rng = np.random.default_rng(seed)
    N = 64
    base = np.float32(2.0 ** -6)
    x_prev = np.zeros((T, K), dtype=np.float32)
    delta = rng.standard_normal((T, K)) * float(base) * 0.3        # PoT 0 .. 1
    delta[:, :n_heavy] = -float(base) * 2.0 ** pot_heavy
    x_t = delta.astype(np.float32)
    w = rng.integers(-127, 128, (K, N)).astype(np.int8)
    w[:n_heavy, 0] = -128
    w[:n_heavy, 1] = 127
    return dict(x_t=x_t, x_prev=x_prev, w=w, w_scale=rng.uniform(1e-3, 1e-2, N).astype(np.float32),
                y_prev=rng.standard_normal((T, N)).astype(np.float32), base=base, k0=2, token_tile=T,
                rows=T, tokens_per_seq=T, K=K, N=N, name=f"w=-128 K={K} PoT={pot_heavy}x{n_heavy}")


@pytest.mark.parametrize("K,pot,n_heavy", [(1024, 14, 1024), (64, 21, 8), (1024, 14, 1016)],
                         ids=["at-2^24", "pot21-at-bound", "just-under"])
def test_int32_bound_with_w_minus_128(dm, K, pot, n_heavy):
    """The product kernel proves a tile exact only when 128·Σ_k 2^PoT_k < 2^31
    (|W| ≤ 128: int8 includes −128).  At Σ 2^PoT = 2^24 a column of −128 makes
    S = +2^31, which int32 cannot hold: that tile must take the exact per-group
    path.  Just under the bound the MFMA path holds S exactly.  Y_t and S are
    compared with the oracle bit for bit."""
    d = w_minus_128_case(K, 32, pot, n_heavy, seed=K + pot + n_heavy)
    codes, tags, hist = fmdq.quantize(d["x_t"], d["x_prev"], 32, d["base"], d["k0"])
    pot_all = digits.pot_of(tags)
    bound = int((1 << pot_all.astype(np.int64)).sum())
    perm, off = fmdq.bucket(tags)
    y, accs = fmdq.linear(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], d["base"], 32,
                          return_acc=True)
    s0 = fmdq.shift_combine(accs[0])
    log(f"case {d['name']}: sum 2^PoT = {bound} (limit {(2 ** 31 - 1) // 128}), "
        f"S[0][0] = {int(s0[0, 0])}, max |S| = {int(np.abs(s0).max())}")
    if n_heavy == K or pot == 21:
        assert bound >= (1 << 24) - (1 << 10) and abs(int(s0[0, 0])) >= (1 << 31) - (1 << 20)
    g = gpu_layer(dm, d, sdump=(0, 1))
    check_integer_stages(g, codes, tags, hist, perm, off, d["name"], d["w"])
    check_s(g["s"], accs, [0], 0, d["name"])
    check_y(g["y"], y, d["y_prev"], d["name"])


def test_timestep_chain_in_place(dm):
    """Three consecutive pairs of config 1's random walk on its first 96 rows,
    each implementation chaining its own cached output."""
    import torch
    y_orc = None
    y_gpu = None
    for pair in (1, 2, 3):
        d = wl.make_inputs(1, "fc1", pair, rows=96)
        d["tokens_per_seq"] = 96
        if y_orc is None:
            y_orc = d["y_prev"].copy()
            y_gpu = d["y_prev"].copy()
        r = fmdq.layer(d["x_t"], d["x_prev"], d["w"], d["w_scale"], y_orc, d["base"],
                       d["token_tile"], d["k0"])
        g = gpu_layer(dm, d, inplace=True, y_prev_np=y_gpu)
        check_y(g["y"], r["y"], y_orc, f"chain pair {pair}")
        y_orc, y_gpu = r["y"], g["y"]


@pytest.mark.parametrize("dynamic", [False, True], ids=["static", "dynamic"])
def test_graph_replay_matches_eager(dm, dynamic):
    """One layer step captured in a HIP graph and replayed three times, with
    eager work and synchronizations between the replays, gives after every
    replay the same output (bit for bit) as the same number of eager steps;
    and the eager steps match the oracle's chained outputs.  The dynamic-base
    step (three more kernels, which reset and finalize the base in device
    memory) is captured the same way."""
    import torch
    dev = torch.device("cuda:0")
    d = wl.make_custom(rows=300, K=1152, N=512, token_tile=32, seed=11, heavy=0.1)
    rows, T = d["rows"], d["token_tile"]
    w = torch.from_numpy(d["w"]).to(dev)
    ws = torch.from_numpy(d["w_scale"]).to(dev)
    x_t = torch.from_numpy(d["x_t"]).to(dev)
    x_p = torch.from_numpy(d["x_prev"]).to(dev)
    layer = dm.FmdqLayer(w, ws, rows, T, float(d["base"]), d["k0"])
    run = (lambda lay, *a, **k: lay.step_dynamic(*a, **k)) if dynamic else \
        (lambda lay, *a, **k: lay.step(*a, **k))
    base = fmdq.dynamic_base(d["x_t"], d["x_prev"], T, d["base"]) if dynamic else d["base"]
    # eager reference: the output after 1, 2, 3 in-place steps
    y_e = torch.from_numpy(d["y_prev"]).to(dev)
    refs = []
    for _ in range(3):
        run(layer, x_t, x_p, y_e)
        refs.append(y_e.cpu().numpy().copy())
    y_orc = d["y_prev"]
    for r in range(3):
        y_orc = fmdq.layer(d["x_t"], d["x_prev"], d["w"], d["w_scale"], y_orc, base, T,
                           d["k0"])["y"]
        np.testing.assert_array_equal(refs[r], y_orc, err_msg=f"eager step {r + 1}")
    # graph: warm up on a side stream, capture one step, replay
    y_g = torch.from_numpy(d["y_prev"]).to(dev)
    scratch = torch.empty_like(y_g)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(layer, x_t, x_p, y_g.clone(), y_out=scratch)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(layer, x_t, x_p, y_g)
    other = dm.FmdqLayer(w, ws, rows, T, float(d["base"]), d["k0"])
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        # eager work between replays, on the same kind of buffers
        run(other, x_p, x_t, scratch)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y_g.cpu().numpy(), refs[r], err_msg=f"graph replay {r + 1}")
        log(f"  graph replay {r + 1}: bit-identical to {r + 1} eager steps")


FULL = [(1, "fc1"), (1, "fc2"), (2, "qkv"), (2, "fc1"), (2, "fc2"), (3, "fc1"), (3, "fc2"),
        (4, "fc1"), (4, "fc2")]


@pytest.mark.parametrize("cfg,layer", FULL, ids=lambda v: str(v))
def test_full_size_workloads(dm, cfg, layer):
    """Full-size workload, pair 1: every integer stage in full; Y_t of every
    token tile against the oracle's whole layer, bit for bit, from both the
    product kernel and the per-group kernel; the product kernel's exact S on
    the last eight tiles (the ragged one included where the workload has one)
    and the per-group kernel's accumulators on the last two."""
    t0 = time.time()
    d = wl.make_inputs(cfg, layer, 1)
    rows, T = d["rows"], d["token_tile"]
    nt = (rows + T - 1) // T
    s_lo = max(0, nt - 8)
    log(f"case config {cfg} {layer}: rows={rows} K={d['K']} N={d['N']} T={T} tiles={nt} "
        f"(inputs {time.time() - t0:.1f}s)")
    g = gpu_layer(dm, d, dbg=(nt - 2, nt), sdump=(s_lo, nt))
    log(f"  gpu done {time.time() - t0:.1f}s")
    codes, tags, hist = fmdq.quantize(d["x_t"], d["x_prev"], T, d["base"], d["k0"])
    perm, off = fmdq.bucket(tags)
    log(f"  oracle quantize+bucket done {time.time() - t0:.1f}s")
    check_integer_stages(g, codes, tags, hist, perm, off, d["name"], d["w"])
    y = par_linear(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], d["base"], T)
    log(f"  oracle linear (all {nt} tiles) done {time.time() - t0:.1f}s")
    check_y(g["y"], y, d["y_prev"], d["name"])
    check_y(g["y_dbg"], y, d["y_prev"], d["name"] + " (per-group kernel)")
    _, accs = fmdq.linear(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], d["base"], T,
                          tiles=range(s_lo, nt), return_acc=True)
    for tau in (nt - 2, nt - 1):
        np.testing.assert_array_equal(g["acc"][tau - (nt - 2)].astype(np.int64), accs[tau],
                                      err_msg=f"group accumulators of tile {tau}")
    check_s(g["s"], accs, range(s_lo, nt), s_lo, d["name"])
    log(f"  done {time.time() - t0:.1f}s")


def par_linear_s(codes, tags, perm, off, w, w_scale, y_prev, base, T):
    """Y of every tile and S of every tile ([n_t][T][N] int64), the oracle's
    linear and shift_combine(group_accumulators) called per tile in parallel
    threads."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    rows, N = y_prev.shape[0], w.shape[1]
    nt = (rows + T - 1) // T
    y = np.array(y_prev, dtype=np.float32, copy=True)
    s_all = np.zeros((nt, T, N), dtype=np.int64)

    def run(tau):
        yy, accs = fmdq.linear(codes, tags, perm, off, w, w_scale, y_prev, base, T, tiles=[tau],
                               return_acc=True)
        return tau, yy, fmdq.shift_combine(accs[tau])

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        for tau, yy, st in ex.map(run, range(nt)):
            r0, r1 = tau * T, min(rows, tau * T + T)
            y[r0:r1] = yy[r0:r1]
            s_all[tau] = st
    return y, s_all


# Shapes large enough for the dispatch to take the ping-pong kernel (T = 32,
# K >= 4096, its 256 x 256 blocks filling at least half of the CUs).
def _random_cases(n: int, seed: int) -> list:
    """Seeded random small shapes across the dispatch: K mostly a multiple of
    16 (the product kernels, partial last chunks included), sometimes not (the
    per-group kernel); T of 16, 32 or 64; ragged tiles; batches of two
    sequences; no, some or all sub-channels heavy; narrow and wide scales."""
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(r.choice([16, 32, 64]))
        K = int(16 * r.integers(1, 130)) if r.random() < 0.8 else int(r.integers(1, 700))
        N = int(4 * r.integers(1, 160))
        two = r.random() < 0.25
        tps = int(T * r.integers(1, 8)) if two else int(r.integers(1, 700))
        rows = 2 * tps if two else tps
        heavy = float(r.choice([0.0, 0.05, 0.3, 1.0]))
        c_range = [(0.5, 8.0), (0.02, 4000.0), (4.0, 8.0)][int(r.integers(0, 3))]
        out.append(dict(rows=rows, K=K, N=N, T=T, seed=200 + i, heavy=heavy, c_range=c_range,
                        tokens_per_seq=tps))
    return out


RANDOM_CASES = _random_cases(48, 2026)


@pytest.mark.parametrize("case", RANDOM_CASES,
                         ids=lambda c: f"{c['rows']}x{c['K']}x{c['N']}-T{c['T']}-s{c['seed']}")
def test_random_shapes_match_oracle(dm, case):
    """Every stage bit for bit against the oracle: codes, tags, histogram,
    perm and offsets, the exact S of the kernel that runs, the per-group
    accumulators, and Y_t of both stage-3 paths."""
    c = dict(case)
    d = wl.make_custom(c.pop("rows"), c.pop("K"), c.pop("N"), c.pop("T"), seed=c.pop("seed"), **c)
    full_compare(dm, d)


def _dense_digit_cases(n: int, seed: int) -> list:
    """Seeded random shapes that send a workgroup through the dense
    second-digit pass: 32-row tiles, N % 16 == 0, K a multiple of 16 up to
    4096, at least three tiles per 128-row block, most sub-channels heavy
    (about half at PoT >= 7), sometimes wide scales (third digits, tiles
    above the int32 bound) and two sequences."""
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        K = int(16 * r.integers(1, 257))
        N = int(16 * r.integers(1, 41))
        two = r.random() < 0.25
        tps = int(32 * r.integers(2, 7)) if two else int(r.integers(65, 520))
        rows = 2 * tps if two else tps
        heavy = float(r.choice([0.6, 1.0]))
        c_range = [(4.0, 8.0), (2.0, 16.0), (3.0, 40.0), (0.02, 4000.0)][int(r.integers(0, 4))]
        out.append(dict(rows=rows, K=K, N=N, T=32, seed=600 + i, heavy=heavy, c_range=c_range,
                        tokens_per_seq=tps))
    return out


DENSE_DIGIT_CASES = _dense_digit_cases(24, 2027)


def _dense_digit_workgroups(d) -> int:
    """Workgroups (128-row blocks) that the two-workgroup kernel sends through
    the dense second-digit pass: more second-digit units (64 channels with
    PoT >= 7 of an eligible tile) than 64-channel chunks."""
    T, K = d["token_tile"], d["K"]
    pot = fmdq.pot_exponent(fmdq.subchannel_max(fmdq.differential(d["x_t"], d["x_prev"]), T), d["base"])
    nt = pot.shape[0]
    elig = [128 * np.sum(2.0 ** pot[t].astype(np.int64)) < 2 ** 31 for t in range(nt)]
    units = [int(np.ceil((pot[t] >= 7).sum() / 64)) if elig[t] else 0 for t in range(nt)]
    return sum(1 for w in range(0, nt, 4) if sum(units[w:w + 4]) > (K + 63) // 64)


@pytest.mark.parametrize("case", DENSE_DIGIT_CASES,
                         ids=lambda c: f"{c['rows']}x{c['K']}x{c['N']}-s{c['seed']}")
def test_dense_digit_shapes_match_oracle(dm, case):
    """Random shapes where some workgroup takes the dense second-digit pass:
    every stage bit for bit against the oracle."""
    c = dict(case)
    d = wl.make_custom(c.pop("rows"), c.pop("K"), c.pop("N"), c.pop("T"), seed=c.pop("seed"), **c)
    n = _dense_digit_workgroups(d)
    log(f"  {n} workgroup(s) through the dense second-digit pass")
    assert n > 0
    full_compare(dm, d)


PP_CASES = [
    dict(rows=2041, K=4096, N=4096, T=32, seed=91, heavy=0.2, c_range=(0.5, 64.0)),      # ragged last tile
    dict(rows=2048, K=4096, N=4100, T=32, seed=92, heavy=0.3, c_range=(0.02, 4000.0)),   # N % 16 != 0, d2
    dict(rows=2048, K=4160, N=4096, T=32, seed=93, heavy=1.0, c_range=(4.0, 8.0)),       # every channel 8-bit
    # two tiles whose first 1024 channels sit at PoT 14: Σ 2^PoT ≥ 2^24, the
    # exact per-group path inside the kernel; every other tile eligible
    dict(rows=2048, K=4096, N=4096, T=32, seed=94, heavy=0.05, c_range=(0.5, 64.0), wide_tiles=(5, 40)),
    # K % 64 = 16 and 48: a partial last dense chunk
    dict(rows=2048, K=4112, N=4096, T=32, seed=95, heavy=0.2, c_range=(0.02, 4000.0)),
    dict(rows=1999, K=4144, N=4100, T=32, seed=96, heavy=0.1, c_range=(0.5, 64.0)),
]


@pytest.mark.parametrize("case", PP_CASES, ids=lambda c: f"{c['rows']}x{c['K']}x{c['N']}-s{c['seed']}")
def test_ping_pong_kernel_matches_oracle(dm, case):
    """The ping-pong stage-3 kernel (taken at these shapes): every integer
    stage, S of every tile and Y_t of every output bit for bit, and the
    per-group accumulators of the last two tiles."""
    t0 = time.time()
    c = dict(case)
    wide = c.pop("wide_tiles", ())
    d = wl.make_custom(c.pop("rows"), c.pop("K"), c.pop("N"), c.pop("T"), seed=c.pop("seed"), **c)
    rows, T = d["rows"], d["token_tile"]
    nt = (rows + T - 1) // T
    for tau in wide:
        x = d["x_prev"][tau * T:(tau + 1) * T, :1024].astype(np.float64)
        d["x_t"][tau * T:(tau + 1) * T, :1024] = (x - float(d["base"]) * 2.0 ** 14).astype(np.float32)
    log(f"case {d['name']} (ping-pong kernel), tiles at the bound: {list(wide)}")
    g = gpu_layer(dm, d, dbg=(nt - 2, nt), sdump=(0, nt))
    codes, tags, hist = fmdq.quantize(d["x_t"], d["x_prev"], T, d["base"], d["k0"])
    perm, off = fmdq.bucket(tags)
    check_integer_stages(g, codes, tags, hist, perm, off, d["name"], d["w"])
    y, s_all = par_linear_s(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], d["base"], T)
    log(f"  oracle done {time.time() - t0:.1f}s")
    np.testing.assert_array_equal(g["s"], s_all, err_msg=f"{d['name']}: S (product kernel)")
    check_y(g["y"], y, d["y_prev"], d["name"])
    check_y(g["y_dbg"], y, d["y_prev"], d["name"] + " (per-group kernel)")
    _, accs = fmdq.linear(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], d["base"], T,
                          tiles=[nt - 2, nt - 1], return_acc=True)
    for tau in (nt - 2, nt - 1):
        np.testing.assert_array_equal(g["acc"][tau - (nt - 2)].astype(np.int64), accs[tau])
    log(f"  done {time.time() - t0:.1f}s")


# Shapes whose stage-3 grid of 128 x 256 blocks is not below the CU count, so
# the two-workgroup kernel keeps its wide blocks (the small cases take the
# 128 x 128 variant): token tiles of 16, 32 and 64 rows, ragged last tiles,
# third digits, and at T = 32 every sub-channel heavy (the masked dense
# second-digit pass).
WIDE_BLOCK_CASES = [
    dict(rows=500, K=256, N=20480, T=16, seed=141, heavy=0.3, c_range=(0.02, 4000.0)),
    dict(rows=500, K=256, N=20480, T=32, seed=142, heavy=1.0, c_range=(4.0, 8.0)),
    dict(rows=520, K=320, N=20480, T=64, seed=143, heavy=0.05, c_range=(0.5, 64.0)),
]
# Grids whose 128 x 256 blocks number fewer than the CUs but whose 128 x 128
# blocks number more (8 x 40 = 320), so that some CUs run two narrow
# workgroups (the small cases give every workgroup a CU of its own).
NARROW4_CASES = [
    dict(rows=1000, K=320, N=5120, T=32, seed=144, heavy=1.0, c_range=(4.0, 8.0)),
    dict(rows=1024, K=256, N=5120, T=16, seed=145, heavy=0.3, c_range=(0.02, 4000.0)),
]


@pytest.mark.parametrize("case", WIDE_BLOCK_CASES + NARROW4_CASES,
                         ids=lambda c: f"{c['rows']}x{c['K']}x{c['N']}-T{c['T']}")
def test_wide_blocks_match_oracle(dm, case):
    """The two-workgroup kernel's 128 x 256 blocks, and its 128 x 128 blocks
    on a grid larger than the CU count: every integer stage, S of every tile
    and Y_t of every output bit for bit, and the per-group accumulators of
    the last two tiles."""
    t0 = time.time()
    c = dict(case)
    d = wl.make_custom(c.pop("rows"), c.pop("K"), c.pop("N"), c.pop("T"), seed=c.pop("seed"), **c)
    rows, T = d["rows"], d["token_tile"]
    nt = (rows + T - 1) // T
    if T == 32:
        assert _dense_digit_workgroups(d) > 0, "the case no longer takes the dense second-digit pass"
    log(f"case {d['name']} (two-workgroup kernel, {'128 x 128 blocks' if d['N'] == 5120 else '128 x 256 blocks'})")
    g = gpu_layer(dm, d, dbg=(nt - 2, nt), sdump=(0, nt))
    codes, tags, hist = fmdq.quantize(d["x_t"], d["x_prev"], T, d["base"], d["k0"])
    perm, off = fmdq.bucket(tags)
    check_integer_stages(g, codes, tags, hist, perm, off, d["name"], d["w"])
    y, s_all = par_linear_s(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], d["base"], T)
    log(f"  oracle done {time.time() - t0:.1f}s")
    np.testing.assert_array_equal(g["s"], s_all, err_msg=f"{d['name']}: S (product kernel)")
    check_y(g["y"], y, d["y_prev"], d["name"])
    check_y(g["y_dbg"], y, d["y_prev"], d["name"] + " (per-group kernel)")
    _, accs = fmdq.linear(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], d["base"], T,
                          tiles=[nt - 2, nt - 1], return_acc=True)
    for tau in (nt - 2, nt - 1):
        np.testing.assert_array_equal(g["acc"][tau - (nt - 2)].astype(np.int64), accs[tau])
    log(f"  done {time.time() - t0:.1f}s")


# Stage 1 without the plain codes and stage 3 on the MFMA kernels: tiles that
# the kernels finish with the exact int64 path (every sub-channel heavy, or a
# tile at the bound), T of 16, 32 and 64, third digits, both kernels.
NO_PLAIN = [
    dict(rows=64, K=8192, N=72, T=32, seed=20, heavy=1.0, c_range=(4.0, 8.0)),
    dict(rows=128, K=8192, N=64, T=64, seed=22, heavy=1.0, c_range=(4.0, 8.0)),
    dict(rows=64, K=8192, N=72, T=16, seed=38, heavy=1.0, c_range=(4.0, 8.0)),
    dict(rows=200, K=1152, N=260, T=16, seed=36, heavy=0.3, c_range=(0.02, 4000.0)),
    dict(rows=300, K=1040, N=264, T=32, seed=28, heavy=0.2, c_range=(0.02, 4000.0)),
    dict(rows=2048, K=4096, N=4096, T=32, seed=94, heavy=0.05, c_range=(0.5, 64.0), wide_tiles=(5, 40)),
]


@pytest.mark.parametrize("case", NO_PLAIN, ids=lambda c: f"{c['rows']}x{c['K']}x{c['N']}-T{c['T']}-s{c['seed']}")
def test_product_path_without_plain_codes(dm, case):
    """No plain-codes buffer anywhere: tags, aligned codes, digit planes,
    histogram and bucket bit-exact; S of every tile and Y_t of every output
    bit for bit against the oracle."""
    c = dict(case)
    wide = c.pop("wide_tiles", ())
    d = wl.make_custom(c.pop("rows"), c.pop("K"), c.pop("N"), c.pop("T"), seed=c.pop("seed"), **c)
    rows, T = d["rows"], d["token_tile"]
    nt = (rows + T - 1) // T
    for tau in wide:
        x = d["x_prev"][tau * T:(tau + 1) * T, :1024].astype(np.float64)
        d["x_t"][tau * T:(tau + 1) * T, :1024] = (x - float(d["base"]) * 2.0 ** 14).astype(np.float32)
    log(f"case {d['name']} without plain codes, tiles at the bound: {list(wide)}")
    g = gpu_layer(dm, d, sdump=(0, nt), plain_codes=False)
    assert "codes" not in g
    codes, tags, hist = fmdq.quantize(d["x_t"], d["x_prev"], T, d["base"], d["k0"])
    perm, off = fmdq.bucket(tags)
    np.testing.assert_array_equal(g["tags"], tags, err_msg=f"{d['name']}: tags")
    digits.check_operands(g["acodes"], g["hcodes"], codes, tags, d["name"])
    np.testing.assert_array_equal(g["hist"].astype(np.int64), hist, err_msg=f"{d['name']}: bit histogram")
    np.testing.assert_array_equal(g["perm"], perm, err_msg=f"{d['name']}: bucket order")
    np.testing.assert_array_equal(g["group_off"], off, err_msg=f"{d['name']}: group offsets")
    y, s_all = par_linear_s(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], d["base"], T)
    np.testing.assert_array_equal(g["s"], s_all, err_msg=f"{d['name']}: S (product kernel)")
    check_y(g["y"], y, d["y_prev"], d["name"])


def test_per_group_kernel_needs_plain_codes(dm):
    """Asking for the group accumulators (the per-group kernel) without the
    plain codes is an error, not a silent fallback."""
    import torch
    dev = torch.device("cuda:0")
    d = wl.make_custom(64, 64, 32, 32, seed=3)
    p = dm.make_params(64, 64, 32, float(d["base"]), d["k0"])
    z = lambda *shape, dt=torch.int8: torch.zeros(shape, dtype=dt, device=dev)
    acc = z(1, 16, 32, 32, dt=torch.int32)
    y = torch.zeros((64, 32), dtype=torch.float32, device=dev)
    with pytest.raises(RuntimeError, match="codes"):
        dm.linear(p, 32, None, z(2, 64, dt=torch.int16), z(2, 65, dt=torch.int32), z(64, 64), z(2, 2, 64, 32),
                  z(64, 32), z(32, 64), torch.ones(32, device=dev), y, y, acc, 0, 1)


CHAIN = [(1, "fc1"), (1, "fc2"), (4, "fc1"), (4, "fc2")]


@pytest.mark.parametrize("cfg,layer", CHAIN, ids=lambda v: str(v))
def test_full_size_chain_in_place(dm, cfg, layer):
    """Timestep pairs 1-3 of the workload's random walk at full rows through
    FmdqLayer.step, Y updated in place (each step's Y_t is the next step's
    Y_{t-1}), each implementation chaining its own output (DSTAR Eq. 1 over
    consecutive steps): Y_t of every step bit for bit."""
    import torch
    dev = torch.device("cuda:0")
    t0 = time.time()
    d = wl.make_inputs(cfg, layer, 1)
    xs = wl.make_walk(cfg, layer, 3)
    rows, T = d["rows"], d["token_tile"]
    log(f"case chain config {cfg} {layer}: rows={rows} K={d['K']} N={d['N']} pairs 1-3 "
        f"(inputs {time.time() - t0:.1f}s)")
    # the timed step's configuration: no plain codes (the MFMA kernels read
    # the aligned codes and digit planes only)
    lay = dm.FmdqLayer(torch.from_numpy(d["w"]).to(dev), torch.from_numpy(d["w_scale"]).to(dev), rows, T,
                       float(d["base"]), d["k0"], d["tokens_per_seq"], plain_codes=False)
    assert lay.codes is None
    y = torch.from_numpy(d["y_prev"]).to(dev)
    y_orc = d["y_prev"]
    for pair in (1, 2, 3):
        lay.step(torch.from_numpy(xs[pair]).to(dev), torch.from_numpy(xs[pair - 1]).to(dev), y)
        torch.cuda.synchronize()
        # the oracle's layer: quantize, bucket, then linear on chunks of tiles
        codes, tags, hist = fmdq.quantize(xs[pair], xs[pair - 1], T, d["base"], d["k0"])
        perm, off = fmdq.bucket(tags)
        y_new = par_linear(codes, tags, perm, off, d["w"], d["w_scale"], y_orc, d["base"], T)
        check_y(y.cpu().numpy(), y_new, y_orc, f"{d['name']} pair {pair}")
        y_orc = y_new
        log(f"  pair {pair} done {time.time() - t0:.1f}s, bits {hist.tolist()}")


# ---------------------------------------------------------------- dynamic base
DYN = [
    dict(rows=96, K=64, N=64, T=32, seed=41),
    dict(rows=70, K=44, N=40, T=32, seed=42),                      # ragged last tile
    dict(rows=128, K=37, N=36, T=64, seed=43),                     # K % 4 != 0: scalar loads
    dict(rows=64, K=128, N=96, T=16, seed=44),
    dict(rows=320, K=256, N=264, T=32, seed=45, heavy=0.2),        # MFMA kernel, digit planes
    dict(rows=192, K=192, N=128, T=64, seed=46, c_range=(0.02, 4000.0)),
]


def dyn_compare(dm, d, what):
    rows, T = d["rows"], d["token_tile"]
    nt = (rows + T - 1) // T
    b = fmdq.dynamic_base(d["x_t"], d["x_prev"], T, d["base"])
    log(f"case {what} rows={rows} K={d['K']} N={d['N']} T={T}: oracle base {float(b)!r}")
    g = gpu_layer(dm, d, dbg=(0, nt), dynamic=True)
    assert g["base"].view(np.uint32)[0] == np.asarray(b, dtype=np.float32).view(np.uint32), \
        f"{what}: base {g['base'][0]!r} != {float(b)!r}"
    codes, tags, hist = fmdq.quantize(d["x_t"], d["x_prev"], T, b, d["k0"])
    perm, off = fmdq.bucket(tags)
    check_integer_stages(g, codes, tags, hist, perm, off, what, d["w"])
    y, accs = fmdq.linear(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], b, T,
                          return_acc=True)
    for tau in range(nt):
        np.testing.assert_array_equal(g["acc"][tau].astype(np.int64), accs[tau],
                                      err_msg=f"{what}: group accumulators of tile {tau}")
    check_s(g["s"], accs, range(nt), 0, what)
    check_y(g["y_dbg"], y, d["y_prev"], what + " (per-group kernel)")
    check_y(g["y"], y, d["y_prev"], what)


@pytest.mark.parametrize("case", DYN, ids=lambda c: f"{c['rows']}x{c['K']}x{c['N']}-T{c['T']}-s{c['seed']}")
def test_dynamic_base_layers_match_oracle(dm, case):
    c = dict(case)
    d = wl.make_custom(c.pop("rows"), c.pop("K"), c.pop("N"), c.pop("T"), seed=c.pop("seed"), **c)
    dyn_compare(dm, d, d["name"] + " dyn")


def test_dynamic_base_special_cases(dm):
    """All-zero Δ keeps the static base; a zero sub-channel is left out; the
    clamp to [2^-100, 2^100] (base only)."""
    import torch
    dev = torch.device("cuda:0")
    d = wl.make_custom(64, 12, 8, 32, seed=47)
    x_t = d["x_t"].copy()
    x_t[32:64, 3] = d["x_prev"][32:64, 3]
    d2 = dict(d, x_t=x_t, name="zero-subchannel")
    dyn_compare(dm, d2, "zero sub-channel dyn")
    d3 = dict(d, x_t=d["x_prev"].copy(), name="zero-delta")
    dyn_compare(dm, d3, "all-zero delta dyn")
    delta = d["x_t"].astype(np.float64) - d["x_prev"].astype(np.float64)
    for scale, expect in ((-130, 2.0 ** -100), (110, 2.0 ** 100)):
        xt = torch.from_numpy((delta * 2.0 ** scale).astype(np.float32)).to(dev)
        xp = torch.zeros_like(xt)
        base = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
        p = dm.make_params(64, 12, 32, float(d["base"]), d["k0"])
        log(f"clamp case 2^{scale}")
        dm.dynamic_base(p, xt, xp, base)
        torch.cuda.synchronize()
        got = base.cpu().numpy()[0]
        orc = fmdq.dynamic_base(xt.cpu().numpy(), xp.cpu().numpy(), 32, d["base"])
        assert got == np.float32(expect) == orc


@pytest.mark.parametrize("cfg,layer", [(1, "fc1"), (2, "fc2")], ids=lambda v: str(v))
def test_dynamic_base_full_size(dm, cfg, layer):
    """Full-size workload with the dynamic base: the base bit for bit, every
    integer stage in full, Y on sampled token tiles."""
    t0 = time.time()
    d = wl.make_inputs(cfg, layer, 1)
    rows, T = d["rows"], d["token_tile"]
    nt = (rows + T - 1) // T
    sample = sorted(set([0, 1, nt // 2, nt - 1]))
    b = fmdq.dynamic_base(d["x_t"], d["x_prev"], T, d["base"])
    log(f"case config {cfg} {layer} dyn: rows={rows} K={d['K']} N={d['N']} base {float(b)!r} "
        f"(static {float(d['base'])!r})")
    g = gpu_layer(dm, d, dynamic=True)
    assert g["base"].view(np.uint32)[0] == np.asarray(b, dtype=np.float32).view(np.uint32)
    codes, tags, hist = fmdq.quantize(d["x_t"], d["x_prev"], T, b, d["k0"])
    perm, off = fmdq.bucket(tags)
    check_integer_stages(g, codes, tags, hist, perm, off, d["name"] + " dyn", d["w"])
    y = fmdq.linear(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], b, T, tiles=sample)
    rows_s = np.concatenate([np.arange(tau * T, min(rows, tau * T + T)) for tau in sample])
    check_y(g["y"][rows_s], y[rows_s], d["y_prev"][rows_s], d["name"] + " dyn")
    log(f"  done {time.time() - t0:.1f}s")


# ------------------------------------------------------------------- GELU / MLP
def ulp_distance(a, b):
    """|a - b| in float32 ulps (both arrays float32; signed zeros are equal)."""
    def ordered(x):
        i = np.asarray(x, dtype=np.float32).view(np.int32).astype(np.int64)
        return np.where(i < 0, -(i & 0x7FFFFFFF), i)
    return np.abs(ordered(a) - ordered(b))


def check_gelu(g_gpu, y, what):
    """GELU is evaluated in float64 on both sides (exp from different
    libraries, each within an ulp of float64) and rounded once to float32, so
    the outputs may differ only where the float64 values straddle a float32
    rounding boundary: by one ulp, rarely."""
    d = ulp_distance(g_gpu, fmdq.gelu(y))
    log(f"  {what}: GELU max {int(d.max())} ulp, identical {int((d == 0).sum())}/{d.size}")
    assert d.max() <= 1, f"{what}: GELU differs by {int(d.max())} ulp"


def test_gelu_kernel(dm):
    import torch
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(61)
    special = np.float32([0.0, -0.0, 1e-30, -1e-30, 1e-45, 30.0, -30.0, 1e30, -1e30, -3.0, -5.0, -10.0,
                          -15.0, -20.0, -40.0, 3.4e38, -3.4e38])
    y = np.concatenate([(rng.standard_normal(100003) * 4).astype(np.float32), special])
    g = torch.full((y.size,), float("nan"), dtype=torch.float32, device=dev)
    dm.gelu(torch.from_numpy(y).to(dev), g)
    torch.cuda.synchronize()
    check_gelu(g.cpu().numpy(), y, "gelu kernel")


@pytest.mark.parametrize("case", [SMALL[0], SMALL[2], SMALL[3], SMALL[5], SMALL[8], SMALL[14]],
                         ids=lambda c: f"{c['rows']}x{c['K']}x{c['N']}-T{c['T']}-s{c['seed']}")
def test_linear_gelu_matches_oracle(dm, case):
    """Stage 3 with the fused GELU: Y_t bit for bit, GELU(Y_t) within an ulp."""
    import torch
    dev = torch.device("cuda:0")
    c = dict(case)
    d = wl.make_custom(c.pop("rows"), c.pop("K"), c.pop("N"), c.pop("T"), seed=c.pop("seed"), **c)
    rows, K, N, T = d["rows"], d["K"], d["N"], d["token_tile"]
    log(f"case {d['name']} (fused GELU)")
    w = torch.from_numpy(d["w"]).to(dev)
    lay = dm.FmdqLayer(w, torch.from_numpy(d["w_scale"]).to(dev), rows, T, float(d["base"]), d["k0"],
                       d["tokens_per_seq"])
    y = torch.from_numpy(d["y_prev"]).to(dev)
    g = torch.full((rows, N), float("nan"), dtype=torch.float32, device=dev)
    lay.step(torch.from_numpy(d["x_t"]).to(dev), torch.from_numpy(d["x_prev"]).to(dev), y, gelu_out=g)
    torch.cuda.synchronize()
    r = fmdq.layer(d["x_t"], d["x_prev"], d["w"], d["w_scale"], d["y_prev"], d["base"], T, d["k0"])
    check_y(y.cpu().numpy(), r["y"], d["y_prev"], d["name"])
    check_gelu(g.cpu().numpy(), r["y"], d["name"])


# Shapes whose stage 3 takes each GELU instantiation of the product kernels:
# 128 x 256 blocks of the two-workgroup kernel (its grid, 4 x 80 workgroups,
# is not below the CU count, so the 128 x 128 variant is not taken), and the
# ping-pong kernel (T = 32, K >= 4096, 8 x 16 blocks of 256 x 256 filling
# half of the CUs).  The small cases above take the 128 x 128 blocks.
GELU_WIDE = [
    dict(rows=512, K=256, N=20480, T=32, seed=131, heavy=0.2, c_range=(0.02, 4000.0)),
    dict(rows=2048, K=4096, N=4096, T=32, seed=132, heavy=0.1, c_range=(0.5, 64.0)),
]


@pytest.mark.parametrize("case", GELU_WIDE, ids=lambda c: f"{c['rows']}x{c['K']}x{c['N']}-s{c['seed']}")
def test_linear_gelu_wide_blocks_match_oracle(dm, case):
    """The fused GELU at the wide-block and ping-pong dispatch: Y_t of every
    output bit for bit (oracle over every tile), GELU(Y_t) within an ulp."""
    import torch
    dev = torch.device("cuda:0")
    t0 = time.time()
    c = dict(case)
    d = wl.make_custom(c.pop("rows"), c.pop("K"), c.pop("N"), c.pop("T"), seed=c.pop("seed"), **c)
    rows, N, T = d["rows"], d["N"], d["token_tile"]
    log(f"case {d['name']} (fused GELU, wide blocks)")
    lay = dm.FmdqLayer(torch.from_numpy(d["w"]).to(dev), torch.from_numpy(d["w_scale"]).to(dev), rows, T,
                       float(d["base"]), d["k0"], d["tokens_per_seq"])
    y = torch.from_numpy(d["y_prev"]).to(dev)
    g = torch.full((rows, N), float("nan"), dtype=torch.float32, device=dev)
    lay.step(torch.from_numpy(d["x_t"]).to(dev), torch.from_numpy(d["x_prev"]).to(dev), y, gelu_out=g)
    torch.cuda.synchronize()
    y_gpu, g_gpu = y.cpu().numpy(), g.cpu().numpy()
    codes, tags, _ = fmdq.quantize(d["x_t"], d["x_prev"], T, d["base"], d["k0"])
    perm, off = fmdq.bucket(tags)
    y_orc = par_linear(codes, tags, perm, off, d["w"], d["w_scale"], d["y_prev"], d["base"], T)
    log(f"  oracle done {time.time() - t0:.1f}s")
    check_y(y_gpu, y_orc, d["y_prev"], d["name"])
    check_gelu(g_gpu, y_orc, d["name"])


def test_mlp_chain_matches_oracle(dm):
    """Three timestep pairs through fc1 (fused GELU) → fc2 of the PixArt-alpha
    MLP at 256 rows: Y1 and Y2 bit for bit, G within an ulp.  The oracle's
    second linear takes the GPU's G (an ulp apart at most), so its integer
    decisions are made on the same inputs."""
    import torch
    dev = torch.device("cuda:0")
    R, T = 256, 32
    d1 = [wl.make_inputs(1, "fc1", p, rows=R) for p in (1, 2, 3)]
    d2 = wl.make_inputs(1, "fc2", 1, rows=R)
    k0 = d1[0]["k0"]
    y1_0, y2_0 = d1[0]["y_prev"], d2["y_prev"]
    # static base of the second linear, profiled on the first step (oracle)
    g0 = fmdq.gelu(y1_0)
    y1_1 = fmdq.layer(d1[0]["x_t"], d1[0]["x_prev"], d1[0]["w"], d1[0]["w_scale"], y1_0, d1[0]["base"],
                      T, k0)["y"]
    base2 = wl.profiled_base(fmdq.gelu(y1_1).astype(np.float64) - g0.astype(np.float64))
    log(f"MLP chain: fc2 base {float(base2)!r}")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    mlp = dm.FmdqMLP(t(d1[0]["w"]), t(d1[0]["w_scale"]), float(d1[0]["base"]), t(d2["w"]),
                     t(d2["w_scale"]), float(base2), R, T, k0, tokens_per_seq=R)
    mlp.start(t(y1_0), t(y2_0))
    torch.cuda.synchronize()
    g_prev = mlp.g_cur.cpu().numpy().copy()
    check_gelu(g_prev, y1_0, "start")
    y1o, y2o = y1_0, y2_0
    for s, d in enumerate(d1):
        mlp.step(t(d["x_t"]), t(d["x_prev"]))
        torch.cuda.synchronize()
        y1g, gg, y2g = mlp.y1.cpu().numpy(), mlp.g_cur.cpu().numpy().copy(), mlp.y2.cpu().numpy()
        r1 = fmdq.layer(d["x_t"], d["x_prev"], d["w"], d["w_scale"], y1o, d["base"], T, k0)
        check_y(y1g, r1["y"], y1o, f"step {s + 1} fc1")
        check_gelu(gg, r1["y"], f"step {s + 1}")
        r2 = fmdq.layer(gg, g_prev, d2["w"], d2["w_scale"], y2o, base2, T, k0)
        check_y(y2g, r2["y"], y2o, f"step {s + 1} fc2")
        log(f"  step {s + 1}: bits fc1 {r1['hist'].tolist()} fc2 {r2['hist'].tolist()}")
        y1o, y2o, g_prev = r1["y"], r2["y"], gg


# ------------------------------------------------------------- 2-bit slice stream
SLICE_CASES = [
    dict(rows=96, K=40, N=8, T=32, seed=71, heavy=0.2, c_range=(0.05, 500.0)),
    dict(rows=70, K=33, N=8, T=32, seed=72, heavy=0.5, c_range=(0.05, 500.0)),    # ragged, odd K
    dict(rows=128, K=64, N=8, T=64, seed=73, heavy=0.3),
    dict(rows=40, K=17, N=8, T=16, seed=74, heavy=0.1),
    dict(rows=64, K=2000, N=8, T=32, seed=75, heavy=1.0, c_range=(4.0, 8.0)),     # every channel 8-bit
]


def gpu_slices(dm, d):
    import torch
    dev = torch.device("cuda:0")
    rows, K, T = d["rows"], d["K"], d["token_tile"]
    nt = (rows + T - 1) // T
    p = dm.make_params(rows, K, T, float(d["base"]), d["k0"], d["tokens_per_seq"])
    codes = torch.full((nt, K, T), 90, dtype=torch.int8, device=dev)
    tags = torch.full((nt, K), 0xEE, dtype=torch.uint8, device=dev)
    dm.quantize(p, torch.from_numpy(d["x_t"]).to(dev), torch.from_numpy(d["x_prev"]).to(dev), codes, tags)
    ent = torch.full((nt, 4 * K), 0x1234, dtype=torch.int32, device=dev)
    sl = torch.full((nt, 4 * K, T // 4), 0xAB, dtype=torch.uint8, device=dev)
    off = torch.full((nt, 23), -3, dtype=torch.int32, device=dev)
    dm.slice_encode(p, codes, tags, ent, sl, off)
    torch.cuda.synchronize()
    return (codes.cpu().numpy(), tags.cpu().numpy(), ent.cpu().numpy().view(np.uint32), sl.cpu().numpy(),
            off.cpu().numpy())


@pytest.mark.parametrize("case", SLICE_CASES, ids=lambda c: f"{c['rows']}x{c['K']}-T{c['T']}-s{c['seed']}")
def test_slice_stream_matches_oracle(dm, case):
    c = dict(case)
    d = wl.make_custom(c.pop("rows"), c.pop("K"), c.pop("N"), c.pop("T"), seed=c.pop("seed"), **c)
    log(f"case {d['name']} (slice stream)")
    codes, tags, ent, sl, off = gpu_slices(dm, d)
    e_o, s_o, off_o = fmdq.slice_encode(codes, tags)
    np.testing.assert_array_equal(off, off_o, err_msg="slice offsets")
    np.testing.assert_array_equal(ent, e_o, err_msg="entries")
    for tau in range(codes.shape[0]):
        E = int(off_o[tau, -1])
        np.testing.assert_array_equal(sl[tau, :E], s_o[tau, :E], err_msg=f"slices of tile {tau}")
    log(f"  entries per tile {off_o[:, -1].tolist()[:8]} ...: identical")


def test_slice_stream_full_workload_rows(dm):
    """The PixArt-alpha fc1 input at 256 rows (8 token tiles, K = 1152)."""
    d = wl.make_inputs(1, "fc1", 1, rows=256)
    codes, tags, ent, sl, off = gpu_slices(dm, d)
    e_o, s_o, off_o = fmdq.slice_encode(codes, tags)
    np.testing.assert_array_equal(off, off_o)
    np.testing.assert_array_equal(ent, e_o)
    for tau in range(codes.shape[0]):
        E = int(off_o[tau, -1])
        np.testing.assert_array_equal(sl[tau, :E], s_o[tau, :E])
    log(f"  slice stream of {codes.shape[0]} tiles identical; entries per tile {off_o[:, -1].tolist()}")
