"""The C ABI library: it loads, exports every entry point the header declares,
agrees with the oracle on the rule constants, and rejects invalid arguments on
the host (no kernel is launched, so these run without a GPU)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dstar_fmdq.h")
SAR_HEADER = os.path.join(ROOT, "include", "dstar_sar.h")


@pytest.fixture(scope="module")
def lib():
    from differential_mixed_precision_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from differential_mixed_precision_amd import build
        build.build()
    return _binding


def _header():
    with open(HEADER) as f:
        return f.read()


def test_library_exports_every_declared_entry_point(lib):
    text = _header()
    declared = set(re.findall(r"^\s*(?:int64_t|int|const char\*)\s+(dstar_fmdq_\w+)\s*\(", text, re.M))
    assert declared == set(lib.SYMBOLS)
    raw = ctypes.CDLL(lib.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), name
    assert lib.load().dstar_fmdq_abi_version() == lib.ABI_VERSION


def test_header_constants_match_oracle_and_binding(lib):
    from oracle import fmdq
    text = _header()
    consts = dict(re.findall(r"#define\s+(DSTAR_\w+)\s+\(?(-?\d+)\)?", text))
    assert int(consts["DSTAR_FMDQ_NUM_TAGS"]) == fmdq.N_TAGS == lib.NUM_TAGS
    assert int(consts["DSTAR_FMDQ_NUM_BINS"]) == fmdq.N_BINS == lib.NUM_BINS
    assert int(consts["DSTAR_FMDQ_TAG_OFFSET"]) == fmdq.TAG_OFF == lib.TAG_OFFSET
    assert int(consts["DSTAR_FMDQ_POT_MAX"]) == fmdq.POT_HI == lib.POT_MAX
    assert int(consts["DSTAR_FMDQ_PREC_SHIFT"]) == fmdq.PREC_SHIFT == lib.PREC_SHIFT
    assert int(consts["DSTAR_FMDQ_ABI_VERSION"]) == lib.ABI_VERSION
    for name, code in (("DSTAR_OK", lib.OK), ("DSTAR_EINVAL", lib.EINVAL), ("DSTAR_ENULL", lib.ENULL),
                       ("DSTAR_EALIGN", lib.EALIGN), ("DSTAR_EUNSUPPORTED", lib.EUNSUPPORTED),
                       ("DSTAR_EHIP", lib.EHIP)):
        assert int(consts[name]) == code


def test_params_struct_layout(lib):
    assert ctypes.sizeof(lib.Params) == 24
    assert [f[0] for f in lib.Params._fields_] == ["rows", "tokens_per_seq", "K", "token_tile",
                                                    "base", "thr0_log2"]


FAKE = 0x10000  # a 64 KiB-aligned address; never dereferenced (calls fail validation first)


def _q(lib, p, x=FAKE, xp=FAKE, codes=FAKE, tags=FAKE, acodes=None, hcodes=None, hist=None):
    L = lib.load()
    return L.dstar_fmdq_quantize(ctypes.byref(p) if p is not None else None, x, xp, codes, tags, acodes,
                                 hcodes, hist, 0)


def _l(lib, p, N=64, codes=FAKE, perm=FAKE, off=FAKE, acodes=None, hcodes=None, w=FAKE, w_t=None,
       ws=FAKE, y0=FAKE, y1=FAKE, dbg=None, lo=0, hi=0, sdbg=None):
    L = lib.load()
    return L.dstar_fmdq_linear(ctypes.byref(p), N, codes, perm, off, acodes, hcodes, w, w_t, ws, y0, y1,
                               dbg, sdbg, lo, hi, 0)


@pytest.mark.parametrize("field,value", [
    ("K", 0), ("K", 65536), ("token_tile", 8), ("token_tile", 48), ("rows", -1),
    ("base", 0.0), ("base", -1.0), ("base", float("nan")), ("base", float("inf")),
    ("base", 2.0 ** -110), ("thr0_log2", 0), ("thr0_log2", 16), ("tokens_per_seq", 0)])
def test_invalid_params_rejected(lib, field, value):
    p = lib.make_params(256, 64, 32, 0.05, 2)
    setattr(p, field, value)
    assert _q(lib, p) == lib.EINVAL
    assert lib.load().dstar_fmdq_last_error().decode()
    L = lib.load()
    assert L.dstar_fmdq_bucket(ctypes.byref(p), FAKE, FAKE, FAKE, 0) == lib.EINVAL
    assert _l(lib, p) == lib.EINVAL
    assert L.dstar_fmdq_dynamic_base(ctypes.byref(p), FAKE, FAKE, FAKE, 0) == lib.EINVAL
    assert L.dstar_fmdq_quantize_dyn(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
                                     0) == lib.EINVAL


def test_sequences_must_tile_evenly(lib):
    p = lib.make_params(2 * 100, 64, 32, 0.05, 2, tokens_per_seq=100)   # 100 % 32 != 0
    assert _q(lib, p) == lib.EINVAL
    p = lib.make_params(250, 64, 32, 0.05, 2, tokens_per_seq=128)       # not a multiple
    assert _q(lib, p) == lib.EINVAL


def test_null_and_alignment_errors(lib):
    L = lib.load()
    assert L.dstar_fmdq_quantize(None, FAKE, FAKE, FAKE, FAKE, None, None, None, 0) == lib.ENULL
    p = lib.make_params(64, 64, 32, 0.05, 2)
    assert _q(lib, p, x=None) == lib.ENULL
    assert _q(lib, p, tags=None) == lib.ENULL
    assert _q(lib, p, x=FAKE + 4) == lib.EALIGN
    assert _q(lib, p, codes=FAKE + 8) == lib.EALIGN
    assert _q(lib, p, hist=FAKE + 2) == lib.EALIGN
    assert _q(lib, p, tags=FAKE + 2) == lib.EALIGN
    assert L.dstar_fmdq_bucket(ctypes.byref(p), FAKE, None, FAKE, 0) == lib.ENULL
    assert L.dstar_fmdq_bucket(ctypes.byref(p), FAKE, FAKE + 1, FAKE, 0) == lib.EALIGN
    assert _l(lib, p, w=None) == lib.ENULL
    assert _q(lib, p, acodes=FAKE + 4, hcodes=FAKE) == lib.EALIGN
    assert _q(lib, p, acodes=FAKE, hcodes=FAKE + 8) == lib.EALIGN
    assert _q(lib, p, acodes=FAKE) == lib.ENULL          # the digit planes come with acodes
    assert _q(lib, p, hcodes=FAKE) == lib.ENULL
    # the plain codes may be left out only when the aligned codes are written
    assert _q(lib, p, codes=None) == lib.ENULL
    assert _q(lib, p, codes=None, acodes=FAKE + 4, hcodes=FAKE) == lib.EALIGN   # past the NULL check
    assert _l(lib, p, codes=None) == lib.ENULL
    assert _l(lib, p, codes=None, acodes=FAKE, hcodes=FAKE, w_t=FAKE + 4) == lib.EALIGN
    assert _l(lib, p, acodes=FAKE + 8, hcodes=FAKE, w_t=FAKE) == lib.EALIGN
    assert _l(lib, p, acodes=FAKE, hcodes=FAKE + 4, w_t=FAKE) == lib.EALIGN
    assert _l(lib, p, acodes=FAKE, hcodes=FAKE, w_t=FAKE + 4) == lib.EALIGN
    assert L.dstar_fmdq_pack_weights(0, 16, FAKE, FAKE, 0) == lib.EINVAL
    assert L.dstar_fmdq_pack_weights(16, 0, FAKE, FAKE, 0) == lib.EINVAL
    assert L.dstar_fmdq_pack_weights(16, 16, None, FAKE, 0) == lib.ENULL
    assert L.dstar_fmdq_pack_weights(16, 16, FAKE, FAKE + 8, 0) == lib.EALIGN
    assert _l(lib, p, y1=FAKE + 4) == lib.EALIGN
    assert _l(lib, p, w=FAKE + 8) == lib.EALIGN
    assert _l(lib, p, N=66) == lib.EINVAL
    assert _l(lib, p, N=0) == lib.EINVAL
    assert _l(lib, p, dbg=FAKE, lo=1, hi=1) == lib.EINVAL
    assert _l(lib, p, dbg=FAKE, lo=0, hi=3) == lib.EINVAL    # 64 rows / 32 = 2 tiles
    assert "debug tile range" in L.dstar_fmdq_last_error().decode()
    assert _l(lib, p, sdbg=FAKE, lo=0, hi=3) == lib.EINVAL   # the S dump shares the range check
    assert _l(lib, p, sdbg=FAKE + 4, lo=0, hi=1) == lib.EALIGN   # int64: 8-byte aligned
    # 2-bit slice stream
    se = lambda q, **kw: L.dstar_fmdq_slice_encode(ctypes.byref(q), kw.get("c", FAKE), FAKE, kw.get("e", FAKE),
                                                   FAKE, kw.get("o", FAKE), 0)
    assert se(p, c=None) == lib.ENULL
    assert se(p, c=FAKE + 4) == lib.EALIGN
    assert se(p, e=FAKE + 2) == lib.EALIGN
    assert se(lib.make_params(64, 16385, 32, 0.05, 2)) == lib.EUNSUPPORTED
    # fused GELU and the stand-alone GELU
    lg = lambda go, y0=FAKE, y1=FAKE: L.dstar_fmdq_linear_gelu(ctypes.byref(p), 64, FAKE, FAKE, FAKE, None, None,
                                                               FAKE, None, FAKE, y0, y1, go, 0)
    assert lg(None) == lib.ENULL
    assert lg(FAKE + 4) == lib.EALIGN
    assert lg(FAKE + 0x1000, y1=FAKE + 0x1000) == lib.EINVAL      # gelu_out aliases y_out
    assert lg(FAKE + 0x1000, y0=FAKE + 0x1000) == lib.EINVAL      # ... or y_prev
    # any shared byte is rejected: one row (64 floats) apart overlaps for 64 rows
    assert lg(FAKE + 0x1000 + 256, y1=FAKE + 0x1000) == lib.EINVAL
    assert lg(FAKE + 0x1000, y0=FAKE + 0x1000 + 256) == lib.EINVAL
    assert "overlaps" in L.dstar_fmdq_last_error().decode()
    assert L.dstar_fmdq_gelu(FAKE, FAKE, -1, 0) == lib.EINVAL
    assert L.dstar_fmdq_gelu(None, FAKE, 8, 0) == lib.ENULL
    assert L.dstar_fmdq_gelu(FAKE + 4, FAKE, 8, 0) == lib.EALIGN
    assert L.dstar_fmdq_gelu(None, None, 0, 0) == lib.OK           # empty: no launch
    # dynamic base and the _dyn stages
    assert L.dstar_fmdq_dynamic_base(ctypes.byref(p), FAKE, FAKE, None, 0) == lib.ENULL
    assert L.dstar_fmdq_dynamic_base(ctypes.byref(p), None, FAKE, FAKE, 0) == lib.ENULL
    assert L.dstar_fmdq_dynamic_base(ctypes.byref(p), FAKE, FAKE, FAKE + 2, 0) == lib.EALIGN
    assert L.dstar_fmdq_dynamic_base(ctypes.byref(p), FAKE + 4, FAKE, FAKE, 0) == lib.EALIGN
    assert L.dstar_fmdq_quantize_dyn(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, None, None, None,
                                     0) == lib.ENULL
    assert L.dstar_fmdq_quantize_dyn(ctypes.byref(p), FAKE + 1, FAKE, FAKE, FAKE, FAKE, None, None,
                                     None, 0) == lib.EALIGN
    assert L.dstar_fmdq_quantize_dyn(ctypes.byref(p), FAKE, None, FAKE, FAKE, FAKE, None, None, None,
                                     0) == lib.ENULL
    assert L.dstar_fmdq_linear_dyn(ctypes.byref(p), None, 64, FAKE, FAKE, FAKE, None, None, FAKE, None,
                                   FAKE, FAKE, FAKE, None, None, 0, 0, 0) == lib.ENULL
    assert L.dstar_fmdq_linear_dyn(ctypes.byref(p), FAKE, 66, FAKE, FAKE, FAKE, None, None, FAKE, None,
                                   FAKE, FAKE, FAKE, None, None, 0, 0, 0) == lib.EINVAL


def test_layer_workspace_and_its_checks(lib):
    """The one-call layer: its workspace size is the sum of the intermediates
    (each rounded up to 256 bytes), and a missing, misaligned or short
    workspace is rejected before any launch."""
    L = lib.load()
    r256 = lambda v: (v + 255) // 256 * 256
    for rows, K, T in ((8192, 1152, 32), (300, 1152, 64), (40, 33, 16)):
        p = lib.make_params(rows, K, T, 0.05, 2)
        nt = (rows + T - 1) // T
        want = (r256(nt * K * T) * 2 + r256(2 * nt * K * T) + r256(nt * K) + r256(2 * nt * K) +
                r256(4 * nt * 65))
        assert lib.layer_workspace_size(p) == want
    bad = lib.make_params(64, 64, 48, 0.05, 2)
    assert L.dstar_fmdq_layer_workspace_size(ctypes.byref(bad)) == lib.EINVAL
    p = lib.make_params(64, 64, 32, 0.05, 2)
    need = lib.layer_workspace_size(p)
    lay = lambda ws, nb, N=64: L.dstar_fmdq_layer(ctypes.byref(p), N, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                  FAKE, None, ws, nb, 0)
    assert lay(None, need) == lib.ENULL
    assert lay(FAKE + 16, need) == lib.EALIGN
    assert lay(FAKE, need - 1) == lib.EINVAL
    assert "needed" in L.dstar_fmdq_last_error().decode()
    assert lay(FAKE, need, N=66) == lib.EINVAL


def test_noalloc_layer_rejects_sizes_above_its_scratch_on_the_host(lib):
    """The no-allocation layer checks its size against the library's scratch
    before any HIP call (so this runs without a GPU)."""
    L = lib.load()
    p = lib.make_params(8192, 4608, 32, 0.05, 2, 4096)      # ~151 MB of intermediates
    assert lib.layer_workspace_size(p) > lib.NOALLOC_MAX_BYTES
    rc = L.dstar_fmdq_layer_noalloc(ctypes.byref(p), 1152, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0)
    assert rc == lib.EINVAL
    assert "scratch" in L.dstar_fmdq_last_error().decode()
    bad = lib.make_params(64, 64, 48, 0.05, 2)
    assert L.dstar_fmdq_layer_noalloc(ctypes.byref(bad), 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                      0) == lib.EINVAL
    text = _header()
    m = re.search(r"#define\s+DSTAR_FMDQ_NOALLOC_MAX_BYTES\s+\((\d+)\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == lib.NOALLOC_MAX_BYTES


def test_empty_input_is_a_no_op(lib):
    p = lib.make_params(0, 64, 32, 0.05, 2, tokens_per_seq=1)
    assert _q(lib, p, x=None, xp=None, codes=None, tags=None) == lib.OK
    L = lib.load()
    assert L.dstar_fmdq_bucket(ctypes.byref(p), None, None, None, 0) == lib.OK
    assert _l(lib, p, codes=None, perm=None, off=None, w=None, ws=None, y0=None, y1=None) == lib.OK


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    from differential_mixed_precision_amd import _binding
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(_binding, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        _binding.load()


def test_library_exports_every_sar_entry_point(lib):
    with open(SAR_HEADER) as f:
        text = f.read()
    declared = set(re.findall(r"^\s*int\s+(dstar_sar_\w+)\s*\(", text, re.M))
    assert declared == set(lib.SAR_SYMBOLS)
    raw = ctypes.CDLL(lib.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), name
    consts = dict(re.findall(r"#define\s+(DSTAR_SAR_\w+)\s+(\d+)", text))
    from oracle import sar
    assert int(consts["DSTAR_SAR_BLOCK"]) == sar.SAR_BLOCK == lib.SAR_BLOCK
    assert int(consts["DSTAR_SAR_TILE"]) == sar.SAR_TILE == lib.SAR_TILE
    assert int(consts["DSTAR_SAR_EXP_FRAC"]) == sar.EXP_FRAC == lib.SAR_EXP_FRAC
    assert int(consts["DSTAR_SAR_PAD"]) == lib.SAR_PAD
    assert int(consts["DSTAR_SAR_MAX_D"]) == lib.SAR_MAX_D
    assert int(consts["DSTAR_SAR_MAX_L"]) == lib.SAR_MAX_L
    assert ctypes.sizeof(lib.SarParams) == 28


def test_sar_rejects_invalid_arguments_on_the_host(lib):
    """Argument checks run before any launch: bad shapes, bases, NULL and
    misaligned pointers, and an impossible nnz."""
    L = lib.load()
    good = lib.make_sar_params(2, 3, 256, 72, 0.01, 2.0 ** -15, 0.125)
    fake = 1 << 20                                  # aligned, never dereferenced on the host
    cases = [
        (lib.make_sar_params(0, 3, 256, 72, 0.01, 1.0, 0.1), lib.EINVAL),
        (lib.make_sar_params(2, 3, 200, 72, 0.01, 1.0, 0.1), lib.EINVAL),
        (lib.make_sar_params(2, 3, 256, 0, 0.01, 1.0, 0.1), lib.EINVAL),
        (lib.make_sar_params(2, 3, 256, 129, 0.01, 1.0, 0.1), lib.EINVAL),
        (lib.make_sar_params(2, 3, 256, 72, 0.0, 1.0, 0.1), lib.EINVAL),
        (lib.make_sar_params(2, 3, 256, 72, 0.01, float("inf"), 0.1), lib.EINVAL),
        (lib.make_sar_params(2, 3, 256, 72, 0.01, 1.0, -1.0), lib.EINVAL),
    ]
    for p, code in cases:
        assert L.dstar_sar_quantize_q(ctypes.byref(p), fake, fake, fake, None) == code
    assert L.dstar_sar_quantize_q(None, fake, fake, fake, None) == lib.ENULL
    assert L.dstar_sar_quantize_q(ctypes.byref(good), None, fake, fake, None) == lib.ENULL
    assert L.dstar_sar_quantize_k(ctypes.byref(good), fake, fake + 8, fake, None) == lib.EALIGN
    assert L.dstar_sar_quantize_v(ctypes.byref(good), fake + 2, fake, fake, None) == lib.EALIGN
    # nnz beyond heads·(L/64)^2 = 48
    assert L.dstar_sar_scores(ctypes.byref(good), fake, fake, 49, fake, fake, fake, fake, fake, fake,
                              None) == lib.EINVAL
    assert L.dstar_sar_pv(ctypes.byref(good), fake, fake, -1, fake, fake, fake, fake, fake, None) == lib.EINVAL
    assert L.dstar_sar_pv(ctypes.byref(good), None, fake, 4, fake, fake, fake, fake, fake, None) == lib.ENULL
    assert "nnz" in L.dstar_fmdq_last_error().decode() or "row_ptr" in L.dstar_fmdq_last_error().decode()
