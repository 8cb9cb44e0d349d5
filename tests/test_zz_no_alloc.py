"""dstar_fmdq_layer_noalloc (through the C ABI): the one-call layer with its
intermediates in the library's own per-GPU scratch array instead of a caller
workspace, for callers that cannot allocate.  Its output must equal dstar_fmdq_layer's (and
the oracle's) on consecutive calls, the second one smaller than the first
(the scratch keeps the first call's contents), and sizes above the scratch
are rejected on the host."""
import ctypes

import numpy as np
import pytest

from gen import workloads as wl
from oracle import fmdq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_mixed_precision_amd as dm
    dm.load()
    return dm


def _noalloc(dm):
    lib = dm._binding.load()
    return lib, lib.dstar_fmdq_layer_noalloc


def _run(dm, d, noalloc):
    import torch
    dev = torch.device("cuda:0")
    rows, K, N, T = d["rows"], d["K"], d["N"], d["token_tile"]
    p = dm.make_params(rows, K, T, float(d["base"]), d["k0"], d["tokens_per_seq"])
    w = torch.from_numpy(d["w"]).to(dev)
    w_t = torch.empty((N, K), dtype=torch.int8, device=dev)
    dm.pack_weights(K, N, w, w_t)
    ws_ = torch.from_numpy(d["w_scale"]).to(dev)
    x_t = torch.from_numpy(d["x_t"]).to(dev)
    x_p = torch.from_numpy(d["x_prev"]).to(dev)
    y0 = torch.from_numpy(d["y_prev"]).to(dev)
    y1 = torch.full((rows, N), float("nan"), dtype=torch.float32, device=dev)
    hist = torch.zeros(4, dtype=torch.int32, device=dev)
    if noalloc:
        lib, f = _noalloc(dm)
        stream = torch.cuda.current_stream().cuda_stream
        rc = f(ctypes.byref(p), N, x_t.data_ptr(), x_p.data_ptr(), w.data_ptr(), w_t.data_ptr(), ws_.data_ptr(),
               y0.data_ptr(), y1.data_ptr(), hist.data_ptr(), stream)
        assert rc == 0, lib.dstar_fmdq_last_error().decode()
    else:
        raw = torch.empty(dm.layer_workspace_size(p) + 256, dtype=torch.uint8, device=dev)
        off = (-raw.data_ptr()) % 256
        dm.layer(p, N, x_t, x_p, w, w_t, ws_, y0, y1, raw[off:off + dm.layer_workspace_size(p)], hist)
    torch.cuda.synchronize()
    return y1.cpu().numpy(), hist.cpu().numpy().astype(np.int64)


def test_noalloc_layer_equals_workspace_layer_on_two_calls(dm):
    cases = [wl.make_custom(300, 1152, 520, 32, seed=81, heavy=0.1, c_range=(0.5, 64.0)),
             wl.make_custom(96, 640, 256, 32, seed=82, heavy=0.3, c_range=(0.02, 4000.0))]
    for d in cases:
        print(f"case {d['name']} (no-alloc layer)", flush=True)
        y_na, h_na = _run(dm, d, noalloc=True)
        y_ws, h_ws = _run(dm, d, noalloc=False)
        np.testing.assert_array_equal(y_na, y_ws, err_msg=f"{d['name']}: no-alloc vs workspace layer")
        np.testing.assert_array_equal(h_na, h_ws)
        r = fmdq.layer(d["x_t"], d["x_prev"], d["w"], d["w_scale"], d["y_prev"], d["base"], d["token_tile"],
                       d["k0"])
        np.testing.assert_array_equal(y_na, r["y"], err_msg=f"{d['name']}: no-alloc vs oracle")
        np.testing.assert_array_equal(h_na, r["hist"])
        print(f"  identical to the workspace layer and the oracle ({y_na.size} outputs)", flush=True)


def test_noalloc_rejects_sizes_above_its_scratch(dm):
    lib, f = _noalloc(dm)
    p = dm.make_params(8192, 4608, 32, 0.05, 2, 4096)      # needs ~151 MB of intermediates
    assert dm.layer_workspace_size(p) > dm._binding.NOALLOC_MAX_BYTES
    fake = 1 << 20
    rc = f(ctypes.byref(p), 1152, fake, fake, fake, fake, fake, fake, fake, None, None)
    assert rc == dm._binding.EINVAL
    assert "scratch" in lib.dstar_fmdq_last_error().decode()
