"""A plain C program uses include/gpb.h and libgpb.so with no torch in the
process: the header compiles as C11, host-side checks behave as documented,
and on the GPU one full layer (plan, clear, scatter, gather) run from C
matches the oracle byte for byte."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import pins
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_consumer", "consumer.c")
LIBDIR = os.path.join(ROOT, "gather_plan_build_amd")
ROCM = "/opt/rocm"


def build_consumer(tmp):
    exe = os.path.join(tmp, "consumer")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROCM, "include"), "-o", exe, SRC,
                    "-L", LIBDIR, "-lgpb", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + LIBDIR, "-Wl,-rpath," + os.path.join(ROCM, "lib")],
                   check=True)
    return exe


def test_header_compiles_as_c_and_host_checks_hold():
    with tempfile.TemporaryDirectory() as tmp:
        exe = build_consumer(tmp)
        r = subprocess.run([exe, "check"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr


def _write_batch(path, b, pool, cur):
    head = [b.bs, b.page_size, b.row_bytes, b.n_pool_pages, b.n_pool_entries,
            b.n_writers, b.staging_cap_pages]
    with open(path, "wb") as f:
        np.asarray(head, "<i4").tofile(f)
        np.asarray(b.prefix_pages, "<i4").tofile(f)
        np.asarray(b.cur_tokens, "<i4").tofile(f)
        np.asarray([len(b.req_pages)], "<i4").tofile(f)
        np.asarray(b.req_pages, "<i4").tofile(f)
        pool.tofile(f)
        cur.tofile(f)


def _read_result(path, b):
    raw = open(path, "rb").read()
    S, T, NCP = np.frombuffer(raw[:12], "<i4")
    bs, npp = b.bs, b.n_pool_pages
    sizes = [bs, 2 * bs, 2 * bs, bs, bs, bs, bs, bs, bs, S, S, S, npp, npp, NCP, T, T, T,
             T, 4 * bs, S - NCP, NCP, T, NCP, NCP, 4 * (S - NCP), 4 * NCP,
             b.n_writers + 1, T, T, NCP]
    at = 12
    plan = {}
    for name, n in zip(oracle.PLAN_FIELDS, sizes):
        plan[name] = np.frombuffer(raw[at:at + 4 * n], "<i4")
        at += 4 * n
    stag_bytes = b.staging_rows_total * b.row_bytes
    staging = np.frombuffer(raw[at:at + stag_bytes], np.uint8).reshape(-1, b.row_bytes)
    at += stag_bytes
    dense = np.frombuffer(raw[at:], np.uint8).reshape(-1, b.row_bytes)
    return plan, staging, dense


@pytest.mark.gpu
@pytest.mark.parametrize("seed", [0, 1])
def test_c_consumer_layer_matches_oracle(orc, seed):
    rng = np.random.default_rng(500 + seed)
    batches = [workloads.make_batch("tiny")] + [
        workloads.random_batch(rng, page_size=16, row_bytes=64, n_writers=2,
                               n_pool_entries=2) for _ in range(3)]
    with tempfile.TemporaryDirectory() as tmp:
        exe = build_consumer(tmp)
        for k, b in enumerate(batches):
            pool, cur = pins.tagged_values(b, seed=seed * 10 + k)
            fin, fout = os.path.join(tmp, "in.bin"), os.path.join(tmp, "out.bin")
            _write_batch(fin, b, pool, cur)
            print("c consumer batch", k, "bs", b.bs, flush=True)
            r = subprocess.run([exe, "run", fin, fout], capture_output=True, text=True,
                               timeout=120)
            assert r.returncode == 0, r.stdout + r.stderr
            assert "per-writer scatters and plan build with clear agree" in r.stdout, r.stdout
            plan, staging, dense = _read_result(fout, b)
            want = oracle.plan_for(b, orc)
            for name in oracle.PLAN_FIELDS:
                assert np.array_equal(plan[name], want[name]), name
            st = np.empty(b.staging_rows_total * b.row_bytes, np.uint8)
            wd, bad = oracle.layer_for(b, want, pool.reshape(-1), cur, st, orc)
            assert not bad
            assert np.array_equal(dense, wd) and np.array_equal(staging, st.reshape(-1, b.row_bytes))
