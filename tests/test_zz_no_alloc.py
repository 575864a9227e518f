"""The one-launch layer for callers that cannot allocate device memory
(gpb_compose_layer_noalloc: staging in the library's static array) against
gpb_compose_layer with a caller-allocated staging region, and against the
oracle, byte for byte.  Two calls in a row, the second on a smaller batch:
the array still holds the first call's rows where the second batch's tail
rows are read back, so a call that skipped its clear would show."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

POISON = 0xA5


def _say(*a):
    print(*a, flush=True)


def _layer_both_ways(gpb, b, orc):
    """Dense of layer 0 through gpb_compose_layer (caller staging) and through
    gpb_compose_layer_noalloc, each into a poisoned buffer, plus the oracle's."""
    pools, curs = workloads.make_values(b, device="cuda")
    meta = gpb.BatchMeta.of(b)
    r = gpb.ComposeRunner(meta, pools, curs)
    r.begin_batch()
    r.dense[0].fill_(POISON)
    r.layer(0)
    dense = torch.full_like(r.dense[0], POISON)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    table = [(pools[0], b.n_pool_pages)] * b.n_pool_entries
    gpb.compose_layer_noalloc(dense, table, b.n_writers, b.staging_cap_pages, r.plan, r.S,
                              r.plan.NCP, curs[0], r.T, b.page_size, b.row_bytes, status)
    torch.cuda.synchronize()
    assert int(r.status.item()) == 0 and int(status.item()) == 0
    want_plan = oracle.plan_for(b, orc)
    staging = np.zeros(b.staging_rows_total * b.row_bytes, np.uint8)
    want, bad = oracle.layer_for(b, want_plan, pools[0].cpu().numpy().reshape(-1),
                                 curs[0].cpu().numpy(), staging, orc)
    assert not bad
    return r.dense[0].cpu().numpy(), dense.cpu().numpy(), want.reshape(-1)


def test_noalloc_layer_matches_the_caller_staging_layer(orc):
    import gather_plan_build_amd as gpb
    big = workloads.make_batch("multi_source")
    small = workloads.make_batch("tiny")
    big_bytes = big.staging_rows_total * big.row_bytes
    small_bytes = small.staging_rows_total * small.row_bytes
    assert small_bytes < big_bytes <= gpb.binding.SCRATCH_BYTES
    for b in (big, small):
        _say("noalloc layer", b.name, "slots", b.n_req_pages, "rows", b.n_cur_tokens,
             "writers", b.n_writers, "staging bytes", b.staging_rows_total * b.row_bytes)
        caller, noalloc, want = _layer_both_ways(gpb, b, orc)
        assert np.array_equal(caller, want), "%s: gpb_compose_layer differs" % b.name
        if not np.array_equal(noalloc, caller):
            rows = np.nonzero((noalloc.reshape(-1, b.row_bytes) !=
                               caller.reshape(-1, b.row_bytes)).any(axis=1))[0]
            raise AssertionError("%s: %d dense rows differ, first %s"
                                 % (b.name, len(rows), rows[:8].tolist()))


def test_noalloc_layer_refuses_staging_beyond_the_array():
    """A geometry whose staging would not fit is refused before any launch:
    the dense buffer keeps its poison."""
    import gather_plan_build_amd as gpb
    b = workloads.make_batch("tiny")
    pools, curs = workloads.make_values(b, device="cuda")
    r = gpb.ComposeRunner(gpb.BatchMeta.of(b), pools, curs)
    r.begin_batch()
    dense = torch.full_like(r.dense[0], POISON)
    slab_bytes = b.page_size * b.row_bytes
    too_many = gpb.binding.SCRATCH_BYTES // slab_bytes + 1
    with pytest.raises(gpb.GpbError) as e:
        gpb.compose_layer_noalloc(dense, [(pools[0], b.n_pool_pages)], 1, too_many, r.plan,
                                  r.S, r.plan.NCP, curs[0], r.T, b.page_size, b.row_bytes)
    assert e.value.code == gpb.binding.ESCRATCH
    torch.cuda.synchronize()
    assert (dense.cpu().numpy() == POISON).all()


def test_noalloc_layer_on_a_side_stream_and_in_a_graph(orc):
    import gather_plan_build_amd as gpb
    b = workloads.make_batch("medium")
    pools, curs = workloads.make_values(b, device="cuda")
    meta = gpb.BatchMeta.of(b)
    r = gpb.ComposeRunner(meta, pools, curs)
    r.begin_batch()
    torch.cuda.synchronize()
    want_plan = oracle.plan_for(b, orc)
    staging = np.zeros(b.staging_rows_total * b.row_bytes, np.uint8)
    want, bad = oracle.layer_for(b, want_plan, pools[0].cpu().numpy().reshape(-1),
                                 curs[0].cpu().numpy(), staging, orc)
    assert not bad
    want = want.reshape(-1)
    table = gpb.Sources([(pools[0], b.n_pool_pages)] * b.n_pool_entries)
    dense = torch.full_like(r.dense[0], POISON)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())

    def call(stream):
        gpb.compose_layer_noalloc(dense, table, b.n_writers, b.staging_cap_pages, r.plan,
                                  r.S, r.plan.NCP, curs[0], r.T, b.page_size, b.row_bytes,
                                  status, stream)

    print("eager call on a side stream", flush=True)
    call(side)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(dense.cpu().numpy(), want)

    print("capture", flush=True)
    graph = torch.cuda.CUDAGraph()
    dense.fill_(POISON)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        call(side)
    torch.cuda.synchronize()
    for k in range(3):
        # eager work between replays: the caller-staging layer over the same
        # pool and a refill of the output with the poison byte
        r.layer(0)
        dense.fill_(POISON)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print("replay", k, flush=True)
        assert int(status.item()) == 0
        assert np.array_equal(dense.cpu().numpy(), want), "replay %d differs" % k
    del graph


def test_noalloc_layer_fills_the_whole_array(orc):
    """Staging of exactly GPB_SCRATCH_BYTES: one slab of 1,024 pages of 64
    rows of 1,024 bytes, 1,023 current pages.  A first batch fills every row
    of the array's top page with current rows; the second batch's last page
    there is partial, so its 50 tail rows must read back as the zeros of the
    second call's clear, not as the first call's rows."""
    import gather_plan_build_amd as gpb
    PS, RB, CAP = 64, 1024, 1024
    assert CAP * PS * RB == gpb.binding.SCRATCH_BYTES
    rng = np.random.default_rng(77)
    n_pool = 4096
    for tail in (0, 50):
        P = np.array([3, 0], np.int32)
        c = np.array([600 * PS + 5, 422 * PS - tail], np.int32)  # 601 + 422 current pages
        n_cur_pages = int(sum((x + PS - 1) // PS for x in c))
        assert n_cur_pages == CAP - 1
        pages = rng.choice(np.arange(1, n_pool), size=int(P.sum()) + n_cur_pages,
                           replace=False).astype(np.int32)
        b = workloads.Batch("full_array", 2, PS, RB, n_pool, 1, 1, CAP, P, c, pages,
                            value_kind="bytes", seed=77 + tail)
        _say("noalloc layer over the whole array, last page short by", tail)
        caller, noalloc, want = _layer_both_ways(gpb, b, orc)
        assert np.array_equal(caller, want)
        assert np.array_equal(noalloc, caller), "tail %d: the layer differs" % tail


def test_noalloc_layer_on_random_small_batches(orc):
    """Random small batches (empty and both-empty requests, page sizes 1 to
    64, rows of 16 to 64 bytes, several pool entries and writers) one after
    another through the array: each equals the caller-staging layer and the
    oracle, whatever the previous batch left in the array."""
    import gather_plan_build_amd as gpb
    import pins
    for i, b in enumerate(pins.random_batches(40, seed=4242)):
        pool_np, cur_np = pins.tagged_values(b)
        pools = [torch.from_numpy(pool_np).cuda()]
        curs = [torch.from_numpy(cur_np).cuda()]
        r = gpb.ComposeRunner(gpb.BatchMeta.of(b), pools, curs)
        r.begin_batch()
        r.dense[0].fill_(POISON)
        r.layer(0)
        dense = torch.full_like(r.dense[0], POISON)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        gpb.compose_layer_noalloc(dense, [(pools[0], b.n_pool_pages)] * b.n_pool_entries,
                                  b.n_writers, b.staging_cap_pages, r.plan, r.S, r.plan.NCP,
                                  curs[0], r.T, b.page_size, b.row_bytes, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0 and int(r.status.item()) == 0, i
        want_plan = oracle.plan_for(b, orc)
        staging = np.zeros(b.staging_rows_total * b.row_bytes, np.uint8)
        want, bad = oracle.layer_for(b, want_plan, pool_np.reshape(-1), cur_np, staging, orc)
        assert not bad
        n = r.S * b.page_size * b.row_bytes
        assert np.array_equal(r.dense[0].cpu().numpy()[:n], want.reshape(-1)), i
        assert np.array_equal(dense.cpu().numpy()[:n], want.reshape(-1)), i
    _say("40 random batches through the array")
