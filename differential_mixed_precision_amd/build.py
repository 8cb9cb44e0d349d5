"""Builds libdstar_fmdq.so (HIP kernels + C ABI) for gfx950 with hipcc.

Usage: python -m differential_mixed_precision_amd.build [-v] [--sanitize]

Objects go to <repo>/_build/, the shared library next to this file.  With
--sanitize the host code (the C ABI's argument checks and launch set-up) is
built with AddressSanitizer and UndefinedBehaviorSanitizer into
<repo>/_build/sanitize/libdstar_fmdq.so; the device code is built as usual.
That library needs the sanitizer runtime preloaded (SANITIZER_RUNTIME) and is
loaded through DSTAR_FMDQ_LIB.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libdstar_fmdq.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no FMA contraction: the quantizer and the epilogue must round exactly
    # as written
    "-ffp-contract=off",
    # keep the compiler away from packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


# host-only sanitizers: each -fsanitize= is scoped to the host compilation
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]
SANITIZE_DIR = os.path.join(BUILD, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, LIB_NAME)


def sanitizer_runtime() -> str | None:
    """The shared ASan runtime of the ROCm clang that compiles the library."""
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    out = SANITIZE_DIR if sanitize else BUILD
    obj = os.path.join(out, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, *(SANITIZE_FLAGS if sanitize else []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs:
        print(msgs, flush=True)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compiles every source under csrc/ and links the shared library (the
    sanitized host build into _build/sanitize/ when `sanitize`)."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    out = SANITIZE_DIR if sanitize else BUILD
    lib_path = SANITIZE_LIB if sanitize else LIB_PATH
    os.makedirs(out, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), srcs))
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
