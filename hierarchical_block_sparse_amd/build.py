"""Build libpyr.so (the C ABI of include/pyr.h) in-tree for gfx950 with hipcc.

Usage: python -m hierarchical_block_sparse_amd.build   (or build() from Python)

`python -m hierarchical_block_sparse_amd.build --sanitize` builds instead
_build/san/libpyr.so: the same library with its host code compiled under
AddressSanitizer and UndefinedBehaviorSanitizer (the device code is built as
usual), for the CPU tests of the C ABI
(load it with PYR_LIBRARY=<path> and the sanitizer runtime preloaded; see
sanitizer_env()).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpyr.so")
SOURCES = ["pyr_api.cpp", "pyramid.hip", "select.hip", "attn.hip", "attn_bwd.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-x", "hip",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]


SAN_LIB = os.path.join(OBJ, "san", "libpyr.so")
# every -fsanitize= goes to the host compilation only
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(x for x in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in x)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libpyr.so; returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        futs = [ex.submit(_run, [HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
                for s, o in zip(SOURCES, objs)]
        for f in futs:
            out = f.result()
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """Compile every source with ASan + UBSan on its host side and link
    _build/san/libpyr.so; returns its path."""
    out_dir = os.path.dirname(SAN_LIB)
    os.makedirs(out_dir, exist_ok=True)
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", *SAN_FLAGS]
    objs = [os.path.join(out_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        futs = [ex.submit(_run, [HIPCC, *flags, "-c", os.path.join(CSRC, s), "-o", o])
                for s, o in zip(SOURCES, objs)]
        for f in futs:
            out = f.result()
            if verbose and out.strip():
                print(out)
    tmp = SAN_LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libsan",
          "-o", tmp, *objs])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def sanitizer_env() -> dict:
    """Environment for a Python process that loads the sanitized library: the
    compiler's ASan runtime preloaded (the interpreter itself is not built with
    it), leak checking off (the interpreter and the HIP runtime keep their
    allocations to the end), every report fatal."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    rt = r.stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        import glob
        found = glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib",
                                       "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
        if not found:
            raise RuntimeError("the ASan runtime of hipcc's clang was not found")
        rt = found[0]
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, PYR_LIBRARY=SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")
    return env


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
