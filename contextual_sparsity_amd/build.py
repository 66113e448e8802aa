"""Builds libdejavu.so (HIP C++ for gfx950) in-tree with hipcc.

    python -m contextual_sparsity_amd.build [--jobs N] [--verbose] [--sanitize]

Sources are compiled in parallel into ``contextual_sparsity_amd/_build/`` and linked
into ``contextual_sparsity_amd/libdejavu.so``.  Every call recompiles everything.

``--sanitize`` builds a separate ``contextual_sparsity_amd/_build_san/libdejavu_san.so``
whose host code (argument validation, workspace planning, launch set-up) carries
AddressSanitizer and UndefinedBehaviorSanitizer checks; the device code is built as
usual.  The sanitizer runtime is not linked in: a process that loads this library
preloads clang's ASan runtime (which also holds UBSan's handlers), e.g. to run the
CPU-side ABI tests against it:

    R=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so)
    DEJAVU_LIB=contextual_sparsity_amd/_build_san/libdejavu_san.so LD_PRELOAD=$R \
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
    python -m pytest tests/test_abi.py
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdejavu.so")
BUILD_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(BUILD_SAN, "libdejavu_san.so")
# host-side checks only (each flag after -Xarch_host, so no device code is instrumented)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]

SOURCES = ["api.cpp", "gemv.hip", "gemv_f16.hip", "gemv_f16_side.hip", "gemv_f32.hip",
           "gemv_f32_side.hip", "gemv_dyn_f16.hip", "gemv_dyn_f32.hip", "gemv_own_f16.hip", "gemv_own_f32.hip",
           "gemv_own_dyn_f16.hip", "gemv_own_dyn_f32.hip", "gemv_mfma.hip", "gather.hip",
           "axpy.hip", "attn.hip", "select.hip", "norms.hip", "lazykv.hip", "misc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdejavu)")


def common_flags():
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        # keep the compiler from forming packed-fp32 VALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    ]


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD_SAN if sanitize else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + (SAN_FLAGS if sanitize else []) + \
        ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def build(jobs: int = 0, verbose: bool = False, sanitize: bool = False) -> str:
    os.makedirs(BUILD_SAN if sanitize else BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), SOURCES))
    out = LIB_SAN if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libdejavu.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="the ASan/UBSan build of the host code (_build_san/libdejavu_san.so)")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose, a.sanitize))
    return 0


if __name__ == "__main__":
    sys.exit(main())
