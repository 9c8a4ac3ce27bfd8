"""The library's host code (argument validation, the ring planner, workspace sizes, error strings)
built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side only (the gfx950 device
code is compiled as usual, with the GPU sanitizer off), and the host ABI tests run against that
build: any out-of-bounds access, use after free, signed overflow or misaligned access on those paths
aborts the run.  Needs no GPU: every call in those tests returns before reaching the GPU."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from blockwise_ring_attention_step_amd import build as ra_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


@pytest.mark.slow
def test_host_abi_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    runtime = _asan_runtime()
    if runtime is None or not os.path.exists(ra_build.hipcc()):
        pytest.skip("hipcc or the clang AddressSanitizer runtime is not installed")
    out = str(tmp_path / "libringattn_host_sanitized.so")
    flags = [f for f in ra_build.HIPCC_FLAGS if f not in ("-O3",)]
    cmd = [ra_build.hipcc(), *flags, "-O1", "-g", "-fno-gpu-sanitize",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan",
           "-I", ra_build.INCLUDE, "-I", ra_build.CSRC,
           *[os.path.join(ra_build.CSRC, s) for s in ra_build.SOURCES], "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    # the host code is instrumented by both sanitizers
    syms = subprocess.run(["nm", "-D", out], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms

    env = dict(os.environ)
    env.update(RING_ATTN_LIBRARY=out, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_host_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    text = run.stdout + run.stderr
    assert run.returncode == 0, text[-4000:]
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert " passed" in text
