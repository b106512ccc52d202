"""The host code of the library (argument checks, planner, cascade split and
decision) under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The library is rebuilt with sanitizer instrumentation on its host half only
(the device code is unchanged and never runs here), then the ABI, planner and
cascade tests of test_abi.py run against that build in a child process with
the sanitizer runtime preloaded.  Any report (heap overflow, use after free,
signed overflow, misaligned access, ...) aborts the child and fails this
test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "paged_kv_varlen_flash_amd", "_build", "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libpagedattn.so")


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(_runtime() is None, reason="clang ASan runtime not installed")
def test_host_code_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from paged_kv_varlen_flash_amd import build
    build.build(out=SAN_LIB, host_flags=("-fsanitize=address", "-fsanitize=undefined",
                                         "-fno-sanitize-recover=undefined",
                                         "-fno-omit-frame-pointer", "-shared-libsan"))
    env = dict(os.environ,
               PA_LIBRARY=SAN_LIB,
               LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1:"
                            "abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail \
        and "runtime error" not in tail, tail
