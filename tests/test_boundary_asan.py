"""The C ABI layer under AddressSanitizer and UBSan, on the CPU.

``exact_tiled_attention_10_amd.build.build_host_asan`` compiles the argument
checks, size queries and launch plans (fa_api.cpp, fa_plan.cpp) with the
sanitizers and the kernel launchers stubbed out; the boundary tests then run
against that library in a child process with the ASan runtime preloaded, so
any out-of-bounds access, use of freed memory or undefined behaviour in the
host code they exercise aborts the run.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    gcc = shutil.which("gcc")
    if gcc is None:
        return None
    path = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_boundary_suite_under_asan_and_ubsan():
    runtime = _asan_runtime()
    if runtime is None or shutil.which("g++") is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    from exact_tiled_attention_10_amd import build as b
    lib = b.build_host_asan()
    env = dict(os.environ)
    env.update(FA_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    assert " passed" in r.stdout, tail
