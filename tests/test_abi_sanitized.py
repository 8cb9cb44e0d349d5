"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with both sanitizers on its host code (argument checks,
workspace carving, launch set-up; the device code is unchanged) into
_build/sanitize/, and tests/test_abi.py runs against it in a child process
with the ASan runtime preloaded.  Every ABI test calls entry points with
arguments the host rejects, so no kernel is launched and no GPU is needed.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from differential_mixed_precision_amd import build as b  # noqa: E402


def _stale(lib: str) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    deps = b.sources() + [os.path.join(b.CSRC, f) for f in os.listdir(b.CSRC) if f.endswith(".h")]
    deps += [os.path.join(b.INCLUDE, f) for f in os.listdir(b.INCLUDE)]
    return any(os.path.getmtime(p) > t for p in deps)


@pytest.fixture(scope="module")
def sanitized_env():
    rt = b.sanitizer_runtime()
    if rt is None or not os.path.exists(b.HIPCC):
        pytest.skip("ROCm clang or its ASan runtime is not installed")
    if _stale(b.SANITIZE_LIB):
        b.build(sanitize=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, DSTAR_FMDQ_LIB=b.SANITIZE_LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env, rt


def _run(cmd, env):
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_sanitized_library_is_the_one_loaded(sanitized_env):
    env, rt = sanitized_env
    probe = ("import os; from differential_mixed_precision_amd import _binding as B; B.load(); "
             "m = open('/proc/self/maps').read(); "
             "print(os.path.realpath(B.LIB_PATH) in m, %r in m)" % os.path.realpath(rt))
    r = _run([sys.executable, "-c", probe], env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.split() == ["True", "True"], r.stdout + r.stderr


def test_abi_tests_pass_under_asan_and_ubsan(sanitized_env):
    env, _ = sanitized_env
    r = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
              os.path.join(ROOT, "tests", "test_abi.py")], env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and " failed" not in out, out[-2000:]


def test_the_sanitizer_is_live(sanitized_env):
    # A caller's params struct cut to 4 bytes (malloc'd, so ASan knows its
    # end): the host check reads past it, and the instrumented build must say so.
    env, _ = sanitized_env
    probe = ("import ctypes; from differential_mixed_precision_amd import _binding as B; lib = B.load(); "
             "libc = ctypes.CDLL(None); libc.malloc.restype = ctypes.c_void_p; raw = libc.malloc(4); "
             "ctypes.memset(raw, 0, 4); "
             "lib.dstar_fmdq_bucket(ctypes.cast(raw, ctypes.POINTER(B.Params)), None, None, None, None)")
    r = _run([sys.executable, "-c", probe], env)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr and "check_params" in r.stderr, r.stderr[-3000:]
