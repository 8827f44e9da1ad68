"""The host runtime under AddressSanitizer and UndefinedBehaviorSanitizer:
libfs.so rebuilt with both on its host code (device code as usual), then the
host-only C-ABI tests (argument validation, struct layout, exports, the
block-table check) run against it in a child process with the ASan runtime
preloaded.  Any sanitizer report fails the test.  CPU only: no kernel runs."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

from kv_cache_injection_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def sanitized_host_command(out: str):
    """hipcc line for libfs.so whose host code carries AddressSanitizer and
    UndefinedBehaviorSanitizer: each -fsanitize follows -Xarch_host, so it
    applies to the host pass only and the device code is built as usual."""
    return [
        build.hipcc(), f"--offload-arch={build.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
        "-fvisibility=hidden", "-fno-omit-frame-pointer",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Xarch_host", "-fsanitize=address",
        "-Xarch_host", "-fsanitize=undefined",
        "-shared-libasan",
        "-I", build.INCLUDE, "-I", build.CSRC,
        "-o", out,
    ] + [os.path.join(build.CSRC, s) for s in build.SOURCES]


def asan_runtime():
    """The toolchain's shared ASan runtime, or None."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_host_runtime_is_clean_under_asan_and_ubsan(tmp_path):
    rt = asan_runtime()
    if rt is None or shutil.which("nm") is None:
        pytest.skip("no shared ASan runtime in the toolchain")
    lib = str(tmp_path / "libfs_san.so")
    res = subprocess.run(sanitized_host_command(lib), cwd=ROOT, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_init" in syms and "__ubsan_handle" in syms, "the build is not instrumented"
    env = dict(os.environ, FS_LIB_PATH=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_abi_host.py"),
                          os.path.join(ROOT, "tests", "test_block_check.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
