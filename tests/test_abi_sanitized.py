"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds a copy of the library with the host side instrumented (the device code
is built as usual), then runs the CPU ABI tests against it in a child process
with the sanitizer runtime preloaded: every validation path, workspace plan
and status string, with out-of-bounds reads, overflows and undefined behaviour
reported as failures."""
import glob
import os
import subprocess
import sys

import pytest

from diffusion_transformer_denoiser_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    for pattern in ("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                    "/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(pattern))
        if hits:
            return hits[-1]
    return None


def test_abi_host_code_under_sanitizers():
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm install")
    lib = build.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", MOSS_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
