"""Host-side logic of bench.py (no GPU): the command-line contract and the
attribution of kernel launches to layers in the rocprofv3 summaries."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_launches_are_attributed_to_the_following_stage3_launch():
    lin = "dstar::(anonymous namespace)::linear_mfma_kernel<32, true, false>(...)"
    q = "dstar::(anonymous namespace)::quantize_kernel<32, 4, 16>(...)"
    b = "dstar::(anonymous namespace)::bucket_ballot_kernel(...)"
    # two steps of two layers: stages 1 and 2 share their grid across layers
    seq = [(1, q, 512), (2, b, 256), (3, lin, 1000),   # fc1
           (4, q, 512), (5, b, 256), (6, lin, 2000),   # fc2
           (7, q, 512), (8, b, 256), (9, lin, 1000),
           (10, q, 512), (11, b, 256), (12, lin, 2000),
           (13, "copyBuffer", 9)]                       # nothing after it
    keys = bench.layer_keys(list(reversed(seq)))       # order of the input does not matter
    assert [keys[i] for i in (1, 2, 3, 7, 8, 9)] == [1000] * 6
    assert [keys[i] for i in (4, 5, 6, 10, 11, 12)] == [2000] * 6
    assert keys[13] is None


def test_stage_algorithmic_bytes_count_each_array_once():
    """The per-launch byte counts are the scope's formulas: stage 1 reads both
    float32 inputs and writes codes and tags (the aligned-operand write is
    reported apart), stage 2 reads tags and writes ids and 17 offsets per
    tile, stage 3 reads codes, W, ids, offsets and w_scale and streams Y."""
    rows, K, N, T = 4608, 3072, 12288, 32
    nt = rows // T
    q = bench.algorithmic("quantize", rows, K, N, T)
    assert q == dict(bytes=8 * rows * K + rows * K + nt * K + 16, ops=0, extra_bytes=0)
    b = bench.algorithmic("bucket", rows, K, N, T)
    assert b["bytes"] == 3 * nt * K + 68 * nt
    lin = bench.algorithmic("linear", rows, K, N, T)
    assert lin["ops"] == 2 * rows * N * K
    assert lin["bytes"] == rows * K + K * N + 2 * nt * K + 68 * nt + 4 * N + 8 * rows * N
    # the table of the scope: FLUX-style fc1 stage 3 moves 506 MB for 348 G ops
    assert round(lin["bytes"] / 1e6) == 506 and round(lin["ops"] / 1e9) == 348


def test_headline_is_the_largest_single_gpu_workload():
    from gen import workloads as wl
    big = max(wl.CONFIGS.values(), key=lambda c: sum(2 * c["rows"] * k * n for k, n in c["layers"].values()))
    assert bench.HEADLINE == big["name"] == "flux-large"


def test_roofline_takes_the_longest_stage():
    kernels = {"quantize@fc1": dict(us_mean=40.0, bound="hbm", gbs=3000.0, tops=0.0, traffic=None,
                                    alg_bytes=1, alg_ops=0),
               "linear@fc1": dict(us_mean=200.0, bound="mfma", gbs=2500.0, tops=1740.0, traffic=123,
                                  alg_bytes=2, alg_ops=3)}
    r = bench.roofline_of(kernels)
    assert r["kernel"] == "linear@fc1" and r["bound"] == "mfma" and r["unit"] == "TOP/s"
    assert abs(r["frac"] - 1740.0 / bench.INT8_PEAK_TOPS) < 1e-12 and r["traffic"] == 123


def test_sq_summary_busy_fraction_from_counters(tmp_path):
    """The stage-3 SQ summary: busy fraction = busy cycles / (1024 SIMDs ·
    GRBM cycles / 8), executed ops = MOPS · 512, against 2·M·K·N of the layer
    that the launch grid names."""
    from gen import workloads as wl
    spec = next(v for v in wl.CONFIGS.values() if v["name"] == "flux-large")
    k, n = spec["layers"]["fc2"]
    grid = bench.layer_grids(spec["rows"], spec["token_tile"], k, n)["linear"]
    alg = 2 * spec["rows"] * k * n
    vals = {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 32 * 1000, "SQ_INSTS_VALU_MFMA_MOPS_I8": alg / 512,
            "SQ_INSTS_VALU_MFMA_I8": 1024 * 1000, "SQ_BUSY_CYCLES": 1, "SQ_WAVE_CYCLES": 1000,
            "SQ_WAIT_ANY": 250, "SQ_ACTIVE_INST_ANY": 500, "GRBM_GUI_ACTIVE": 8 * 64000}
    d = tmp_path / "pmc"
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Grid_Size,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n")
        for disp in (1, 2):
            for c, v in vals.items():
                f.write(f'{disp},{grid},"void dstar::(anonymous namespace)::linear_pp_kernel<32, true, false>'
                        f'(dstar::LinearArgs, int, int)",{c},{v},0,100000\n')
    out = bench.write_sq_summary(str(d), "linear", "flux-large", out_dir=str(tmp_path))
    row = [l for l in open(out) if l.startswith("| `linear_pp_kernel")][0]
    cells = [c.strip() for c in row.strip().strip("|").split("|")]
    assert cells[1].startswith("fc2") and cells[3] == "2" and cells[4] == "100.0"
    assert cells[6] == "32.0" and cells[7] == "**0.500**"          # 32000 busy of 64000 per SIMD
    assert cells[9] == "1.000"                                        # executed = algorithmic
    assert cells[12] == "0.250" and cells[13] == "0.500"


def test_counter_readings_are_keyed_by_code_not_comments():
    src = ('int f(int x) { // doubles x\n'
           '  /* a block\n     comment */ return 2 * x;\n'
           '}\n\n'
           'const char* s = "a // b /* c */";\n'
           "char q = '\"';  // a quote\n")
    assert bench.code_only(src) == ('int f(int x) {\n   return 2 * x;\n}\n'
                                    'const char* s = "a // b /* c */";\n'
                                    "char q = '\"';")
    # a comment edit keeps the key; a code edit changes it
    assert bench.code_only(src.replace("doubles x", "twice x")) == bench.code_only(src)
    assert bench.code_only(src.replace("2 * x", "3 * x")) != bench.code_only(src)
    # every stage's sources hash to a short hex key
    for stage in bench.KERNEL_SRC:
        h = bench.src_sha(stage)
        assert len(h) == 16 and int(h, 16) >= 0
