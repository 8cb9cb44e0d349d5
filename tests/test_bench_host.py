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
    rows, K, N, T = 8192, 1152, 4608, 32
    nt = rows // T
    q = bench.algorithmic("quantize", rows, K, N, T)
    assert q == dict(bytes=8 * rows * K + 2 * nt * T * K + nt * K + 16, ops=0)
    lin = bench.algorithmic("linear", rows, K, N, T)
    assert lin["ops"] == 2 * rows * N * K
    assert lin["bytes"] == nt * T * K + K * N + 2 * nt * K + 260 * nt + 4 * N + 8 * rows * N
