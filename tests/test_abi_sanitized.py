"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

libgpb.so is rebuilt into a temporary directory with the sanitizers on the
host pass only (each -fsanitize= after -Xarch_host; the gfx950 device code is
built as usual), and the host-side ABI tests run against it in a child
pytest with clang's ASan runtime preloaded: argument validation, plan sizing
and the pointer-table checks then run instrumented.  No call here reaches a
kernel launch."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "gather_plan_build_amd", "csrc")


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_host_abi_checks_pass_under_asan_and_ubsan():
    runtime = _clang_asan_runtime()
    if runtime is None:
        pytest.skip("no clang AddressSanitizer runtime under /opt/rocm/llvm")
    with tempfile.TemporaryDirectory() as tmp:
        so = os.path.join(tmp, "libgpb_san.so")
        cmd = ["hipcc", "--offload-arch=gfx950", "-mcode-object-version=5", "-O1", "-g",
               "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all",
               "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", so]
        cmd += sorted(glob.glob(os.path.join(CSRC, "*.hip")))
        subprocess.run(cmd, check=True, capture_output=True)
        env = dict(os.environ, GPB_LIB=so, LD_PRELOAD=runtime,
                   ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                            os.path.join(HERE, "test_abi_host.py")],
                           env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
