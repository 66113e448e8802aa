"""The host code of the library (argument validation, workspace planning, launch set-up)
under AddressSanitizer and UndefinedBehaviorSanitizer: the sanitizer build of the library
(`python -m contextual_sparsity_amd.build --sanitize`) runs the CPU-side ABI tests in a
child process with clang's ASan runtime preloaded.  Any sanitizer report fails the run
(UBSan halts on its first error; leak detection is off, the interpreter's own allocations
would report)."""
import os
import subprocess
import sys

import pytest

from contextual_sparsity_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm's clang is needed for the sanitizer runtime")
def test_abi_under_asan_and_ubsan():
    lib = build.build(sanitize=True)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_" in syms and "__ubsan_handle_" in syms  # the host code is instrumented
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True, check=True).stdout.strip()
    assert os.path.exists(rt), rt
    env = dict(os.environ, DEJAVU_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
