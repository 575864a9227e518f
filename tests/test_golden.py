"""The stored tiny-workload values (tests/golden/tiny_compose.json, written
by tests/golden/make_golden.py from the oracle) against the oracle as it
stands now (CPU) and against the HIP path (GPU)."""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import oracle
import pins
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "tiny_compose.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _check_plan(g, pl, n_pool_pages):
    for k, v in g["plan"].items():
        assert np.array_equal(np.asarray(pl[k]), np.asarray(v, np.int32)), k
    for name in ("page_inverse", "staging_page_inverse"):
        want = np.full(n_pool_pages, -1, np.int32)
        for p, s in g[name + "_set"].items():
            want[int(p)] = s
        assert np.array_equal(np.asarray(pl[name]), want), name


def test_oracle_reproduces_the_stored_values():
    g = _golden()
    b = workloads.make_batch("tiny")
    assert b.req_pages.tolist() == g["batch"]["req_pages"]
    pl = oracle.plan_for(b)
    _check_plan(g, pl, b.n_pool_pages)
    pool, cur = pins.tagged_values(b)
    staging = np.zeros(b.staging_rows_total * b.row_bytes, np.uint8)
    dense, _ = oracle.layer_for(b, pl, pool.reshape(-1), cur, staging)
    assert hashlib.sha256(dense.tobytes()).hexdigest() == g["dense_sha256"]
    assert hashlib.sha256(staging.tobytes()).hexdigest() == g["staging_sha256"]


@pytest.mark.gpu
def test_hip_path_reproduces_the_stored_values():
    import gather_plan_build_amd as gpb
    g = _golden()
    b = workloads.make_batch("tiny")
    pool, cur = pins.tagged_values(b)
    r = gpb.ComposeRunner(gpb.BatchMeta.of(b), [torch.from_numpy(pool).cuda()],
                          [torch.from_numpy(cur).cuda()])
    r.run(1)
    torch.cuda.synchronize()
    _check_plan(g, {k: v.cpu().numpy() for k, v in r.plan.t.items()}, b.n_pool_pages)
    dense = r.dense_of(0).cpu().numpy()
    staging = r.staging_of(0).cpu().numpy()
    assert hashlib.sha256(dense.tobytes()).hexdigest() == g["dense_sha256"]
    assert hashlib.sha256(staging.tobytes()).hexdigest() == g["staging_sha256"]
