"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

gpb_oracle.c is built with gcc -fsanitize=address,undefined (host code only;
nothing here touches a GPU) into a temporary directory, and every pin of
tests/pins.py runs against it in a child process with the ASan runtime
preloaded.  Any out-of-bounds access, use after free, signed overflow or
misaligned access in the oracle aborts the child."""
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "gpb_oracle.c")

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, pins
pins.run_all(oracle.Oracle({lib!r}), n_random=40)
print("SANITIZED PINS OK", flush=True)
"""


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_pass_under_asan_and_ubsan():
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    with tempfile.TemporaryDirectory() as tmp:
        so = os.path.join(tmp, "liboracle_san.so")
        subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-shared",
                        "-fPIC", "-o", so, SRC], check=True)
        env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        code = CHILD.format(root=ROOT, tests=HERE, lib=so)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                           text=True, timeout=600)
    assert r.returncode == 0 and "SANITIZED PINS OK" in r.stdout, \
        (r.stdout[-2000:] + r.stderr[-4000:])
