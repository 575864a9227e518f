"""The oracle against its pins (CPU only): brute force on tagged rows, the
closed form, torch/numpy special cases, the hand-derived tiny example and the
fail-fast cases.  Page citations are in tests/pins.py and oracle/."""
import numpy as np
import pytest

import oracle
import pins
import workloads


def test_tiny_worked_example(orc):
    pins.pin_tiny_worked(orc)


def test_validation_fail_fast(orc):
    pins.pin_validation(orc)


def test_sentinels_and_out_of_range(orc):
    pins.pin_sentinels(orc)


@pytest.mark.parametrize("seed", range(6))
def test_random_batches(orc, seed):
    for b in pins.random_batches(80, seed=seed):
        pins.check_batch(orc, b)


@pytest.mark.parametrize("W,NP", [(2, 1), (3, 2), (8, 8), (32, 32)])
def test_multi_writer_batches(orc, W, NP):
    for b in pins.random_batches(25, seed=100 + W, n_writers=W, n_pool_entries=NP):
        pins.check_batch(orc, b)


def test_page_edges(orc):
    """Current lengths 63/64/65 and 0, both-zero requests, bs = 0."""
    for c in ([63, 64, 65], [0, 0, 0], [1, 0, 128], []):
        bs = len(c)
        P = np.array([2, 0, 1][:bs], np.int32)
        c = np.array(c, np.int32)
        n = int(P.sum() + ((c + 63) // 64).sum())
        pages = np.arange(1, n + 1, dtype=np.int32)[::-1].copy()
        b = workloads.Batch("edge", bs, 64, 32, max(n + 1, 2), 1, 1,
                            workloads.staging_cap_for(int(c.sum()), bs), P, c, pages)
        pins.check_batch(orc, b)


def test_capacity_exact_fit(orc):
    """CAP = 1 + current pages is the smallest staging that fits."""
    P = np.array([1, 0], np.int32)
    c = np.array([64, 70], np.int32)           # 1 + 2 = 3 current pages
    pages = np.array([4, 2, 7, 3], np.int32)
    for cap, ok in ((4, True), (3, False)):
        rc = orc.validate(2, 64, 16, 8, 1, 1, cap, P, c, pages)
        assert (rc == oracle.OK) == ok
        if ok:
            pins.check_batch(orc, workloads.Batch("fit", 2, 64, 16, 8, 1, 1, cap, P, c, pages))


def test_named_workload_metadata(orc):
    """The five workloads are valid batches with the stated structure."""
    for name in workloads.CONFIGS:
        b = workloads.make_batch(name)
        assert orc.validate(b.bs, b.page_size, b.row_bytes, b.n_pool_pages,
                            b.n_pool_entries, b.n_writers, b.staging_cap_pages,
                            b.prefix_pages, b.cur_tokens, b.req_pages) == oracle.OK
    t = workloads.make_batch("traced")
    assert t.bs == 12 and t.n_cur_tokens == 44600
    assert np.all(t.prefix_pages <= 512)
    o = workloads.make_batch("opaque")
    assert o.row_bytes == 656 and o.bs == 32
    assert np.all(o.prefix_pages[0::3] == 0) and np.all(o.cur_tokens[1::3] == 0)
    m = workloads.make_batch("multi_source")
    assert m.n_pool_entries == 8 and m.n_writers == 8


def test_medium_plan_against_brute_force(orc):
    """The medium workload's plan (16K-page pool) through the geometry pins,
    with small rows so the tagged arenas stay small."""
    b = workloads.make_batch("medium")
    b.row_bytes = 16
    pins.check_batch(orc, b)


def test_multi_source_plan(orc):
    b = workloads.make_batch("multi_source")
    b.row_bytes = 16
    pins.check_batch(orc, b)
