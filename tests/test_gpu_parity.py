"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, byte
for byte, on the five workloads at full size and on random small batches.

Every comparison is exact: the path moves integers and opaque bytes only.
Inputs are seeded (workloads/); the oracle reads host copies of the very
bytes the GPU reads."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
import pins
import workloads

pytestmark = pytest.mark.gpu


def _gpb():
    import gather_plan_build_amd as gpb
    return gpb


def _say(*a):
    print(*a, flush=True)


def _runner(batch, pools, curs):
    gpb = _gpb()
    return gpb.ComposeRunner(gpb.BatchMeta.of(batch), pools, curs)


def _host(t):
    return t.cpu().numpy()


def _check_plan(batch, r, orc):
    assert int(r.plan.status.item()) == 0, "plan kernels flagged their input"
    want = oracle.plan_for(batch, orc)
    for k in oracle.PLAN_FIELDS:
        got = _host(r.plan.t[k])
        assert np.array_equal(got, want[k]), "plan array %s differs" % k
    return want


def _oracle_layer(batch, want_plan, pool_np, cur_np, orc):
    staging = np.full(batch.staging_rows_total * batch.row_bytes, 0xCD, np.uint8)
    dense, bad = oracle.layer_for(batch, want_plan, pool_np.reshape(-1),
                                  cur_np.reshape(-1, batch.row_bytes), staging, orc)
    assert not bad
    return dense, staging.reshape(-1, batch.row_bytes)


def _check_layer(batch, r, layer, want_plan, pools_np, curs_np, orc, check_staging=True):
    k = layer % len(pools_np)
    dense, staging = _oracle_layer(batch, want_plan, pools_np[k], curs_np[k], orc)
    got = _host(r.dense_of(layer))
    assert got.shape == dense.shape
    if not np.array_equal(got, dense):
        bad_rows = np.nonzero((got != dense).any(axis=1))[0]
        raise AssertionError("layer %d: %d dense rows differ, first %s"
                             % (layer, len(bad_rows), bad_rows[:8].tolist()))
    if check_staging:
        assert np.array_equal(_host(r.staging_of(layer)), staging), \
            "layer %d: staging differs" % layer


def _status(r):
    return int(r.status.item())


POISON = 0xA5


def _run_poisoned(r, n_layers, two_launch=False):
    """The batch as bench.py runs it (plan build with the staging clear, then
    each layer's scatter and gather, in one launch or in two), with the dense
    half of each of the last two layers filled with a sentinel byte just
    before that layer runs.  A dense byte the gather fails to write then
    shows as a mismatch instead of passing on the identical bytes an earlier
    layer left in the same half."""
    r.begin_batch()
    for layer in range(n_layers):
        if layer >= n_layers - 2:
            r.dense[layer % 2].fill_(POISON)
        if two_launch:
            r.layer_two_launch(layer)
        else:
            r.layer(layer)


def test_ragged_tails_stay_inside_their_ranges(orc):
    """Pages whose chunk count is not a multiple of a workgroup's unit (656-
    and 48-byte rows) and a scatter whose last workgroup runs past the last
    row: every byte beyond the output range keeps its guard value."""
    gpb = _gpb()
    rng = np.random.default_rng(21)
    for PS, RB in ((64, 656), (3, 48), (1, 16)):
        n_pages, n_slots = 6, 5
        pool_np = rng.integers(0, 256, (n_pages * PS, RB), dtype=np.uint8)
        pool = torch.from_numpy(pool_np).cuda()
        guard = 1 << 20
        out = torch.full((n_slots * PS * RB + guard,), 0x5A, dtype=torch.uint8, device="cuda")
        owner = torch.zeros(n_slots, dtype=torch.int32, device="cuda")
        src = torch.tensor([5, 1, 4, 2, 3], dtype=torch.int32, device="cuda")
        gpb.compose_gather(out, [(pool, n_pages)], owner, src, n_slots, PS, RB)
        torch.cuda.synchronize()
        h = _host(out)
        assert (h[n_slots * PS * RB:] == 0x5A).all(), "gather wrote past its pages"
        want = pool_np.reshape(n_pages, -1)[[5, 1, 4, 2, 3]].reshape(-1)
        assert np.array_equal(h[:n_slots * PS * RB], want)

        n_rows, n_stag = 7, 9
        cur_np = rng.integers(0, 256, (n_rows, RB), dtype=np.uint8)
        rows = np.array([8, 0, 2, 7, 1, 5, 6], np.int32)
        stag = torch.full((n_stag * RB + guard,), 0x5A, dtype=torch.uint8, device="cuda")
        gpb.current_row_scatter(stag, n_stag, torch.from_numpy(rows).cuda(),
                                torch.from_numpy(cur_np).cuda(), n_rows, RB)
        torch.cuda.synchronize()
        h = _host(stag)
        assert (h[n_stag * RB:] == 0x5A).all(), "scatter wrote past the staging"
        want = np.full((n_stag, RB), 0x5A, np.uint8)
        want[rows] = cur_np
        assert np.array_equal(h[:n_stag * RB].reshape(n_stag, RB), want)
        _say("guard ok", PS, RB)


@pytest.mark.parametrize("name", workloads.CONFIGS)
def test_plan_matches_oracle(orc, name):
    b = workloads.make_batch(name)
    _say("plan", name, "bs", b.bs, "slots", b.n_req_pages, "tokens", b.n_cur_tokens)
    gpb = _gpb()
    p = gpb.Plan(gpb.BatchMeta.of(b)).build()
    torch.cuda.synchronize()
    want = oracle.plan_for(b, orc)
    for k in oracle.PLAN_FIELDS:
        assert np.array_equal(_host(p.t[k]), want[k]), "plan array %s differs" % k


def test_tiny_layer_byte_exact(orc):
    b = workloads.make_batch("tiny")
    pools, curs = workloads.make_values(b, device="cuda")
    r = _runner(b, pools, curs)
    _run_poisoned(r, 1)
    torch.cuda.synchronize()
    want = _check_plan(b, r, orc)
    _check_layer(b, r, 0, want, [_host(p) for p in pools], [_host(c) for c in curs], orc)
    assert _status(r) == 0


@pytest.mark.parametrize("name", ["medium", "multi_source"])
def test_single_layer_workloads(orc, name):
    b = workloads.make_batch(name)
    _say(name, "slots", b.n_req_pages, "tokens", b.n_cur_tokens)
    pools, curs = workloads.make_values(b, device="cuda")
    r = _runner(b, pools, curs)
    _run_poisoned(r, b.n_layers)
    torch.cuda.synchronize()
    want = _check_plan(b, r, orc)
    pools_np, curs_np = [_host(p) for p in pools], [_host(c) for c in curs]
    _check_layer(b, r, 0, want, pools_np, curs_np, orc)
    assert _status(r) == 0


@pytest.mark.parametrize("name", ["traced", "opaque"])
def test_multi_layer_workloads(orc, name):
    """Full-size workloads: the first four layers one at a time (every pool
    rotation), then the whole layer loop as bench.py runs it, checking the
    last two layers (both parity halves)."""
    b = workloads.make_batch(name)
    _say(name, "layers", b.n_layers, "slots", b.n_req_pages, "tokens", b.n_cur_tokens)
    pools, curs = workloads.make_values(b, device="cuda")
    pools_np = [_host(p) for p in pools]
    curs_np = [_host(c) for c in curs]
    r = _runner(b, pools, curs)
    r.begin_batch()
    torch.cuda.synchronize()
    want = _check_plan(b, r, orc)
    for layer in range(4):
        r.dense[layer % 2].fill_(POISON)
        r.layer(layer)
        torch.cuda.synchronize()
        _check_layer(b, r, layer, want, pools_np, curs_np, orc)
        _say("  layer", layer, "ok")
    for two in (False, True):
        _run_poisoned(r, b.n_layers, two_launch=two)
        torch.cuda.synchronize()
        for layer in (b.n_layers - 2, b.n_layers - 1):
            _check_layer(b, r, layer, want, pools_np, curs_np, orc)
            _say("  layer", layer, "two launches" if two else "one launch", "ok")
    for layer, fused in ((0, False), (1, True)):
        _check_split(b, r, layer, want, pools_np[layer % len(pools_np)],
                     curs_np[layer % len(curs_np)], orc, fused_fill=fused)
        _say("  split layer", layer, "fused fill" if fused else "scatter", "ok")
    for layer in (2, 3):
        _check_one_launch(b, r, layer, want, pools_np[layer % len(pools_np)],
                          curs_np[layer % len(curs_np)], orc)
        _say("  one-launch layer and fused consume", layer, "ok")
    _check_layer_fill(b, r, 1, want, pools_np[1 % len(pools_np)], curs_np[1 % len(curs_np)],
                      orc)
    _say("  one-launch layer with fused fill ok")
    assert _status(r) == 0


def _check_split(batch, r, layer, want_plan, pool_np, cur_np, orc, fused_fill):
    """Prefetch split on the GPU (prefix gather, then scatter or fused fill,
    then the current gather) against the oracle: dense and staging equal the
    one-shot layer; with the fused fill, the pool rows of the current tokens
    hold them afterwards and no other pool row changed."""
    dense, staging = _oracle_layer(batch, want_plan, pool_np, cur_np, orc)
    h = layer % 2
    r.dense[h].fill_(0xEE)
    r.gather_prefix(layer)
    torch.cuda.synchronize()
    got = _host(r.dense_of(layer))
    PS = batch.page_size
    for s in want_plan["current_slots"]:
        assert (got[s * PS:(s + 1) * PS] == 0xEE).all(), "prefix gather wrote a current slot"
    if fused_fill:
        pool_before = pool_np.reshape(-1, batch.row_bytes)
        pool_after = pool_before.copy()
        st = np.zeros(batch.staging_rows_total * batch.row_bytes, np.uint8)
        assert not orc.fill(st, want_plan["staging_rows"], pool_after.reshape(-1),
                            want_plan["pool_locs"], cur_np, batch.row_bytes)
        r.fill(layer)
    else:
        r.scatter(layer)
    r.gather_current(layer)
    torch.cuda.synchronize()
    assert np.array_equal(_host(r.dense_of(layer)), dense), "split dense differs"
    assert np.array_equal(_host(r.staging_of(layer)), staging), "split staging differs"
    if fused_fill:
        k = layer % len(r.pools)
        assert np.array_equal(_host(r.pools[k]).reshape(-1, batch.row_bytes), pool_after), \
            "fused fill pool differs"
        r.pools[k].copy_(torch.from_numpy(pool_np.reshape(r.pools[k].shape)))


def _check_one_launch(batch, r, layer, want_plan, pool_np, cur_np, orc):
    """The layer as two launches (gpb_current_row_scatter, then
    gpb_compose_gather) and in one (gpb_compose_layer), and the split with
    its consume half in one launch (prefix records, then
    gpb_compose_consume), each on a cleared staging half and a poisoned dense
    half, against the oracle's layer."""
    dense, staging = _oracle_layer(batch, want_plan, pool_np, cur_np, orc)
    h = layer % 2
    for run in (r.layer_two_launch, r.layer_fused):
        r.staging[h].zero_()
        r.dense[h].fill_(POISON)
        run(layer)
        torch.cuda.synchronize()
        assert np.array_equal(_host(r.dense_of(layer)), dense), \
            "%s: dense differs" % run.__name__
        assert np.array_equal(_host(r.staging_of(layer)), staging), \
            "%s: staging differs" % run.__name__
    r.staging[h].zero_()
    r.dense[h].fill_(POISON)
    r.gather_prefix(layer)
    r.consume_fused(layer)
    torch.cuda.synchronize()
    assert np.array_equal(_host(r.dense_of(layer)), dense), "fused consume dense differs"
    assert np.array_equal(_host(r.staging_of(layer)), staging), "fused consume staging differs"


def _check_layer_ahead(batch, r, layer, want_plan, pool_np, cur_np, orc, fill=False):
    """The layer-ahead launch (gpb_compose_layer_ahead, or with ``fill``
    gpb_compose_layer_ahead_fill) on one batch whose layers share one pool
    and one set of current rows: after layer l's prefix gather, one launch
    consumes layer l into its half and gathers layer l + 1's prefix pages
    into the other half.  Layer l's half and its staging equal the oracle's
    layer; the other half holds the oracle's prefix pages, and its current
    slots keep their poison.  With the fill, the pool holds each current row
    at its pool row and no other pool byte changed (restored afterwards)."""
    assert len(r.pools) == 1 and len(r.curs) == 1
    dense, staging = _oracle_layer(batch, want_plan, pool_np, cur_np, orc)
    h = layer % 2
    r.staging[h].zero_()
    r.dense[h].fill_(POISON)
    r.dense[1 - h].fill_(POISON)
    r.gather_prefix(layer)
    (r.ahead_fill if fill else r.ahead)(layer)
    torch.cuda.synchronize()
    if fill:
        pool_after = pool_np.reshape(-1, batch.row_bytes).copy()
        st = np.zeros(batch.staging_rows_total * batch.row_bytes, np.uint8)
        assert not orc.fill(st, want_plan["staging_rows"], pool_after.reshape(-1),
                            want_plan["pool_locs"], cur_np, batch.row_bytes)
        assert np.array_equal(_host(r.pools[0]).reshape(-1, batch.row_bytes), pool_after), \
            "layer-ahead with fill: pool differs"
        r.pools[0].copy_(torch.from_numpy(pool_np.reshape(r.pools[0].shape)))
    assert np.array_equal(_host(r.dense_of(layer)), dense), "layer-ahead: consumed half differs"
    assert np.array_equal(_host(r.staging_of(layer)), staging), "layer-ahead: staging differs"
    nxt = _host(r.dense_of(layer + 1))
    PS = batch.page_size
    cur = np.zeros(len(nxt) // PS if PS else 0, bool)
    cur[want_plan["current_slots"]] = True
    rows_cur = np.repeat(cur, PS)
    assert np.array_equal(nxt[~rows_cur], dense[~rows_cur]), "layer-ahead: prefix pages differ"
    assert (nxt[rows_cur] == POISON).all(), "layer-ahead: wrote a current slot of the next half"


def _check_layer_fill(batch, r, layer, want_plan, pool_np, cur_np, orc):
    """The one-launch layer with the fused fill: dense and staging equal the
    oracle's layer; the pool holds each current row at its pool row and no
    other pool byte changed (the oracle's fill); the pool is restored
    afterwards."""
    dense, staging = _oracle_layer(batch, want_plan, pool_np, cur_np, orc)
    pool_after = pool_np.reshape(-1, batch.row_bytes).copy()
    st = np.zeros(batch.staging_rows_total * batch.row_bytes, np.uint8)
    assert not orc.fill(st, want_plan["staging_rows"], pool_after.reshape(-1),
                        want_plan["pool_locs"], cur_np, batch.row_bytes)
    h, k = layer % 2, layer % len(r.pools)
    r.staging[h].zero_()
    r.dense[h].fill_(POISON)
    r.layer_fill(layer)
    torch.cuda.synchronize()
    assert np.array_equal(_host(r.dense_of(layer)), dense), "layer with fill: dense differs"
    assert np.array_equal(_host(r.staging_of(layer)), staging), \
        "layer with fill: staging differs"
    assert np.array_equal(_host(r.pools[k]).reshape(-1, batch.row_bytes), pool_after), \
        "layer with fill: pool differs"
    r.pools[k].copy_(torch.from_numpy(pool_np.reshape(r.pools[k].shape)))


def _check_consume_fill(batch, r, layer, want_plan, pool_np, cur_np, orc):
    """The prefix records, then the consume with the fused fill
    (gpb_compose_consume_fill): dense, staging and pool as the oracle's
    layer and fill; the pool is restored afterwards."""
    dense, staging = _oracle_layer(batch, want_plan, pool_np, cur_np, orc)
    pool_after = pool_np.reshape(-1, batch.row_bytes).copy()
    st = np.zeros(batch.staging_rows_total * batch.row_bytes, np.uint8)
    assert not orc.fill(st, want_plan["staging_rows"], pool_after.reshape(-1),
                        want_plan["pool_locs"], cur_np, batch.row_bytes)
    h, k = layer % 2, layer % len(r.pools)
    r.staging[h].zero_()
    r.dense[h].fill_(POISON)
    r.gather_prefix(layer)
    r.consume_fill(layer)
    torch.cuda.synchronize()
    assert np.array_equal(_host(r.dense_of(layer)), dense), "consume with fill: dense differs"
    assert np.array_equal(_host(r.staging_of(layer)), staging), \
        "consume with fill: staging differs"
    assert np.array_equal(_host(r.pools[k]).reshape(-1, batch.row_bytes), pool_after), \
        "consume with fill: pool differs"
    r.pools[k].copy_(torch.from_numpy(pool_np.reshape(r.pools[k].shape)))


def _check_writer_scatters(batch, r, layer, want_plan, pool_np, cur_np, orc):
    """The scatter run as W writers, each copying its own rows (in its list
    order) into its own slab, then one gather: staging and dense equal the
    single scatter's, i.e. the oracle's."""
    dense, staging = _oracle_layer(batch, want_plan, pool_np, cur_np, orc)
    h = layer % 2
    own = r.writer_rows_of(layer)
    assert [int(x.shape[0]) for x in own] == \
        np.diff(want_plan["writer_offsets"]).tolist()
    r.staging[h].zero_()
    r.dense[h].fill_(POISON)
    r.scatter_writers(layer, own)
    r.gather(layer)
    torch.cuda.synchronize()
    assert np.array_equal(_host(r.staging_of(layer)), staging), "per-writer staging differs"
    assert np.array_equal(_host(r.dense_of(layer)), dense), "per-writer dense differs"


def _random_case(orc, b, layers=2):
    pool_np, cur_np = pins.tagged_values(b)
    pools = [torch.from_numpy(pool_np).cuda()]
    curs = [torch.from_numpy(cur_np).cuda()]
    r = _runner(b, pools, curs)
    _run_poisoned(r, layers)
    torch.cuda.synchronize()
    want = _check_plan(b, r, orc)
    for layer in range(max(0, layers - 2), layers):
        _check_layer(b, r, layer, want, [pool_np], [cur_np], orc)
    _check_split(b, r, layers, want, pool_np, cur_np, orc, fused_fill=False)
    _check_split(b, r, layers + 1, want, pool_np, cur_np, orc, fused_fill=True)
    _check_one_launch(b, r, layers, want, pool_np, cur_np, orc)
    _check_writer_scatters(b, r, layers + 1, want, pool_np, cur_np, orc)
    _check_layer_fill(b, r, layers, want, pool_np, cur_np, orc)
    _check_layer_ahead(b, r, layers + 1, want, pool_np, cur_np, orc)
    _check_layer_ahead(b, r, layers, want, pool_np, cur_np, orc, fill=True)
    _check_consume_fill(b, r, layers + 1, want, pool_np, cur_np, orc)
    assert _status(r) == 0


@pytest.mark.parametrize("name,consume", [("traced", "fused"), ("opaque", "fused"),
                                          ("traced", "scatter"), ("medium", "fill"),
                                          ("traced", "one_stream"), ("opaque", "one_stream"),
                                          ("medium", "one_stream"), ("traced", "one_stream_fill"),
                                          ("opaque", "one_stream_fill")])
def test_layer_ahead_schedule(orc, name, consume):
    """The whole batch with the layer-ahead prefetch.  On two streams (default
    priority): layer l + 1's prefix gather runs on a side stream while layer
    l is consumed on the main stream, ordered only by events.  On one stream
    ("one_stream"): one launch per layer holds layer l's consume and layer
    l + 1's prefix gather ("one_stream_fill": the consume also stores the
    current rows in the layer's pool, which no prefix page read shares).
    Every layer's dense half is poisoned just before its prefix gather is
    issued; checked layers are copied out right after
    their consume (before the half goes to layer l + 2) and compared with the
    oracle: the first four layers, a middle pair and the last pair."""
    b = workloads.make_batch(name)
    L = b.n_layers
    _say("pipelined", name, consume, "layers", L)
    pools, curs = workloads.make_values(b, device="cuda")
    pools_np = [_host(p) for p in pools]
    curs_np = [_host(c) for c in curs]
    r = _runner(b, pools, curs)
    checked = sorted({l for l in (0, 1, 2, 3, L // 2, L // 2 + 1, L - 2, L - 1)
                      if 0 <= l < L})
    snaps = {}
    stag = {}

    def poison(l, side):
        with torch.cuda.stream(side):
            r.dense[l % 2].fill_(POISON)

    def keep(l, stream):
        if l in checked:
            with torch.cuda.stream(stream):
                snaps[l] = r.dense_of(l).clone()
                stag[l] = r.staging_of(l).clone()

    main = torch.cuda.current_stream()
    if consume.startswith("one_stream"):
        r.run_layer_ahead(L, main, before_prefetch=poison, after_consume=keep,
                          fill=consume.endswith("fill"))
    else:
        side = torch.cuda.Stream()
        r.run_pipelined(L, main, side, consume=consume, before_prefetch=poison,
                        after_consume=keep)
    torch.cuda.synchronize()
    want = _check_plan(b, r, orc)
    for l in checked:
        k = l % len(pools_np)
        dense, staging = _oracle_layer(b, want, pools_np[k], curs_np[k], orc)
        got = _host(snaps[l])
        if not np.array_equal(got, dense):
            bad_rows = np.nonzero((got != dense).any(axis=1))[0]
            raise AssertionError("pipelined layer %d: %d dense rows differ, first %s"
                                 % (l, len(bad_rows), bad_rows[:8].tolist()))
        assert np.array_equal(_host(stag[l]), staging), "pipelined layer %d staging" % l
        _say("  layer", l, "ok")
    assert _status(r) == 0


@pytest.mark.parametrize("name", ["multi_source", "medium"])
def test_writer_scatters_full_size(orc, name):
    """The full-size batch with the scatter split over its writers (8 on the
    multi-source table): byte-exact staging and dense."""
    b = workloads.make_batch(name)
    pools, curs = workloads.make_values(b, device="cuda")
    r = _runner(b, pools, curs)
    r.begin_batch()
    torch.cuda.synchronize()
    want = _check_plan(b, r, orc)
    _check_writer_scatters(b, r, 0, want, _host(pools[0]), _host(curs[0]), orc)
    _check_one_launch(b, r, 1, want, _host(pools[0]), _host(curs[0]), orc)
    assert _status(r) == 0


def test_shared_plan_must_match_the_batch(orc):
    """A twin format may share a plan only if the batch metadata, the table
    layout and the staging capacity are the same; the row size may differ."""
    gpb = _gpb()
    b = workloads.make_batch("tiny")
    pools, curs = workloads.make_values(b, device="cuda")
    tok = _runner(b, pools, curs)
    rb = 144
    ipools, icurs = workloads.make_values(b, device="cuda", row_bytes=rb, value_kind="bytes")
    ok = gpb.BatchMeta(b.bs, b.page_size, rb, b.n_pool_pages, b.n_pool_entries, b.n_writers,
                       b.staging_cap_pages, b.prefix_pages, b.cur_tokens, b.req_pages)
    gpb.ComposeRunner(ok, ipools, icurs, plan=tok.plan)
    bad = gpb.BatchMeta(b.bs, b.page_size, rb, b.n_pool_pages, b.n_pool_entries,
                        b.n_writers, b.staging_cap_pages + 1, b.prefix_pages, b.cur_tokens,
                        b.req_pages)
    with pytest.raises(ValueError):
        gpb.ComposeRunner(bad, ipools, icurs, plan=tok.plan)


def test_one_launch_layer_reports_a_table_that_breaks_the_layout(orc):
    """The one-launch layer reads each current page back at the address the
    table gives; a table whose staging entries are not the staging the rows
    are written to is reported (GPB_STATUS_LAYER_MISMATCH), while the same
    call with the plan's layout reports nothing.  Either way the current
    pages hold the bytes at the table's address: read through the staging
    region's resource when that address lies in the staging region (here its
    second half, which the call does not write), through the table entry's
    otherwise (a separate buffer); prefix pages and the scatter are as the
    oracle's."""
    gpb = _gpb()
    b = workloads.make_batch("tiny")
    pools, curs = workloads.make_values(b, device="cuda")
    r = _runner(b, pools, curs)
    r.begin_batch()
    torch.cuda.synchronize()
    want_plan = _check_plan(b, r, orc)
    want_dense, want_staging = _oracle_layer(b, want_plan, _host(pools[0]), _host(curs[0]), orc)
    cur_slots = _host(r.plan.t["current_slots"])
    page_rows = np.concatenate([np.arange(s * b.page_size, (s + 1) * b.page_size)
                                for s in cur_slots])
    prefix_rows = np.setdiff1d(np.arange(r.S * b.page_size), page_rows)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    good = r.tables[(0, 0)]
    gpb.compose_layer(r.dense[0], good, r.plan, r.S, r.plan.NCP, r.staging[0],
                      r.staging_rows_total, curs[0], r.T, r.ps, r.rb, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(_host(r.dense_of(0)), want_dense)

    slab = b.staging_cap_pages * b.page_size * b.row_bytes
    elsewhere = torch.full_like(r.staging[0], 0x5A)
    r.staging[1].fill_(0x3C)
    second = r.staging[1].data_ptr()
    pool_entries = [(pools[0], b.n_pool_pages)] * b.n_pool_entries
    cases = [("a separate buffer", 0x5A, r.staging[0], r.staging_rows_total,
              [(elsewhere.data_ptr() + w * slab, b.staging_cap_pages)
               for w in range(b.n_writers)]),
             ("the staging region's second half", 0x3C, r.staging_all,
              2 * r.staging_rows_total,
              [(second + w * slab, b.staging_cap_pages) for w in range(b.n_writers)])]
    for what, byte, staging, n_staging_rows, slabs in cases:
        _say("layer with the staging entries in", what)
        r.staging_all.zero_()
        r.staging[1].fill_(0x3C)
        r.dense[0].fill_(POISON)
        status.zero_()
        bad = gpb.Sources(pool_entries + slabs)
        gpb.compose_layer(r.dense[0], bad, r.plan, r.S, r.plan.NCP, staging, n_staging_rows,
                          curs[0], r.T, r.ps, r.rb, status)
        torch.cuda.synchronize()
        assert int(status.item()) == gpb.STATUS_LAYER_MISMATCH, what
        got = _host(r.dense_of(0))
        assert (got[page_rows] == byte).all(), what
        assert np.array_equal(got[prefix_rows], want_dense[prefix_rows]), what
        assert np.array_equal(_host(r.staging_of(0)), want_staging), what


def test_records_out_of_range_are_skipped(orc):
    """A record whose slot is outside the dense buffer is skipped and
    flagged; the others are gathered."""
    gpb = _gpb()
    PS, RB = 2, 32
    rng = np.random.default_rng(14)
    pool_np = rng.integers(1, 256, (6 * PS, RB), dtype=np.uint8)
    pool = torch.from_numpy(pool_np).cuda()
    dense = torch.full((4 * PS, RB), 0x33, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rec = torch.tensor([[2, 0, 3, 0], [9, 0, 1, 0], [-1, 0, 2, 0], [0, 0, 1, 0],
                        [3, 0, -1, 0]], dtype=torch.int32, device="cuda")
    gpb.compose_gather_records(dense, [(pool, 6)], rec, 5, 4, PS, RB, status)
    torch.cuda.synchronize()
    h = _host(dense).reshape(4, PS, RB)
    want = np.full((4, PS, RB), 0x33, np.uint8)
    want[2] = pool_np[3 * PS:4 * PS]
    want[0] = pool_np[1 * PS:2 * PS]
    want[3] = 0
    assert np.array_equal(h, want)
    assert int(status.item()) == gpb.STATUS_BAD_DESCRIPTOR


@pytest.mark.parametrize("seed", range(4))
def test_random_small_batches(orc, seed):
    """Edge-heavy random batches: empty and both-zero requests, current
    lengths at page edges, page sizes 1..64, rows of 16..64 bytes, up to 3
    pool entries and writers."""
    for i, b in enumerate(pins.random_batches(60, seed=1000 + seed)):
        _random_case(orc, b)
    _say("seed", seed, "done")


def test_random_larger_geometries(orc):
    """300 seeded random batches of larger geometries through every layer
    path: up to 40 requests, many of them empty on one side, pages of 1 to
    64 rows, rows of 16 to 4,096 bytes, up to 8 pool entries and 8 writers,
    spare staging pages."""
    rng = np.random.default_rng(2026)
    done = 0
    while done < 300:
        ps = int(rng.choice([1, 2, 3, 4, 8, 16, 32, 64]))
        rb = int(rng.choice([16, 32, 48, 144, 320, 336, 656, 1024, 1152, 2064, 4096]))
        bs = int(rng.integers(0, 41))
        P = rng.integers(0, 12, bs).astype(np.int32)
        P[rng.random(bs) < 0.3] = 0
        c = rng.integers(0, 5 * ps + 1, bs).astype(np.int32)
        c[rng.random(bs) < 0.3] = 0
        need = int(P.sum() + ((c + ps - 1) // ps).sum())
        n_pool = need + 1 + int(rng.integers(0, 200))
        if n_pool * ps * rb > (64 << 20):
            continue
        pages = rng.choice(np.arange(1, n_pool), need, replace=False).astype(np.int32)
        np_, w = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        cap = workloads.staging_cap_for(int(c.sum()), bs, ps) + int(rng.integers(0, 4))
        _random_case(orc, workloads.Batch("larger", bs, ps, rb, n_pool, np_, w, cap, P, c,
                                          pages))
        done += 1
    _say("300 larger random batches byte-exact")


def test_many_requests_past_the_lds_stage(orc):
    """bs = 1500 exceeds the requests staged in LDS (1024): the plan kernels
    search the bases in global memory."""
    rng = np.random.default_rng(3)
    bs = 1500
    P = rng.integers(0, 3, bs).astype(np.int32)
    c = rng.choice([0, 1, 15, 16, 17, 40], bs).astype(np.int32)
    PS = 16
    n = int(P.sum() + ((c + PS - 1) // PS).sum())
    pages = rng.choice(np.arange(1, n + 100), n, replace=False).astype(np.int32)
    b = workloads.Batch("many", bs, PS, 32, n + 100, 2, 3,
                        workloads.staging_cap_for(int(c.sum()), bs, PS), P, c, pages)
    _random_case(orc, b)


# 336-byte rows (21 chunks) are the smallest whose scatter workgroups fetch
# their staging rows as scalars; 320-byte rows (20 chunks) take the per-lane path
@pytest.mark.parametrize("ps,rb", [(1, 16), (2, 4096 + 16), (64, 656), (64, 1152), (3, 48),
                                   (5, 336), (5, 320)])
def test_row_and_page_geometry(orc, ps, rb):
    rng = np.random.default_rng(ps * 7 + rb)
    for b in [workloads.random_batch(rng, page_size=ps, row_bytes=rb, max_pool=40)
              for _ in range(6)]:
        _random_case(orc, b)


def test_two_host_threads_on_two_streams(orc):
    """The library keeps no global state: two host threads, each driving its
    own batch on its own stream (default priority), interleave their plan
    builds, clears, scatters and gathers, and both results match the
    oracle."""
    import threading
    rng = np.random.default_rng(77)
    batches = [workloads.random_batch(rng, max_bs=8, max_pool=200, page_size=16,
                                      row_bytes=1152) for _ in range(2)]
    cases = []
    for b in batches:
        pool_np, cur_np = pins.tagged_values(b)
        r = _runner(b, [torch.from_numpy(pool_np).cuda()], [torch.from_numpy(cur_np).cuda()])
        cases.append((b, r, pool_np, cur_np, torch.cuda.Stream()))
    torch.cuda.synchronize()
    errors = []

    def drive(case):
        b, r, _, _, st = case
        try:
            with torch.cuda.stream(st):
                for it in range(3):
                    r.begin_batch(st)
                    for layer in range(4):
                        if it == 2 and layer >= 2:
                            r.dense[layer % 2].fill_(POISON)
                        r.layer(layer, st)
            st.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=drive, args=(c,)) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for b, r, pool_np, cur_np, _ in cases:
        want = _check_plan(b, r, orc)
        for layer in (2, 3):
            _check_layer(b, r, layer, want, [pool_np], [cur_np], orc)
        assert _status(r) == 0


@st.composite
def _valid_batches(draw):
    """Well-formed small batches of every geometry the kernels distinguish:
    row sizes on both sides of the scalar-row threshold (21 chunks), pages of
    1 to 64 rows, 1 to 4 pool entries and writers, spare staging pages."""
    ps = draw(st.sampled_from([1, 2, 4, 16, 64]))
    rb = draw(st.sampled_from([16, 48, 144, 320, 336, 656, 1152]))
    bs = draw(st.integers(0, 8))
    P = np.array([draw(st.integers(0, 4)) for _ in range(bs)], np.int32)
    c = np.array([draw(st.integers(0, 3 * ps)) for _ in range(bs)], np.int32)
    need = int(P.sum() + ((c + ps - 1) // ps).sum())
    n_pool = need + 1 + draw(st.integers(0, 20))
    rng = np.random.default_rng(draw(st.integers(0, 2 ** 32 - 1)))
    pages = rng.choice(np.arange(1, n_pool), need, replace=False).astype(np.int32)
    np_, w = draw(st.integers(1, 4)), draw(st.integers(1, 4))
    cap = workloads.staging_cap_for(int(c.sum()), bs, ps) + draw(st.integers(0, 2))
    return workloads.Batch("hypothesis", bs, ps, rb, n_pool, np_, w, cap, P, c, pages)


@settings(max_examples=40, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(_valid_batches())
def test_property_random_batches_byte_exact(orc, b):
    """Hypothesis-drawn batches (fixed derivation, so every run draws the
    same ones): plan, two layers and both prefetch-split variants byte-exact
    against the oracle."""
    _random_case(orc, b)


def _full_table_batch():
    """The largest pointer table the ABI takes: 32 pool entries and 32 staging
    slabs (64 entries), with 51 current pages dealt round robin over the 32
    writers, 4-token pages and 48-byte rows."""
    rng = np.random.default_rng(64)
    P = np.array([3, 0, 2, 5, 1, 0, 4, 2], np.int32)
    c = np.array([37, 20, 0, 9, 64, 3, 17, 41], np.int32)
    PS, RB, NP, W = 4, 48, 32, 32
    need = int(P.sum() + ((c + PS - 1) // PS).sum())
    n_pool = need + 40
    pages = rng.choice(np.arange(1, n_pool), size=need, replace=False).astype(np.int32)
    cap = workloads.staging_cap_for(int(c.sum()), len(P), PS)
    return workloads.Batch("full_table", len(P), PS, RB, n_pool, NP, W, cap, P, c, pages)


def test_full_pointer_table(orc):
    b = _full_table_batch()
    assert b.n_pool_entries + b.n_writers == 64
    assert int(((b.cur_tokens + b.page_size - 1) // b.page_size).sum()) > b.n_writers
    _say("full table: 64 entries, slots", b.n_req_pages, "tokens", b.n_cur_tokens)
    _random_case(orc, b)


def _owner_arenas(b, pool):
    """One pool arena per pool entry, as each rank would hold its own pool:
    arena e keeps the pages p with p mod NP == e and holds the sentinel byte
    everywhere else, so a page read through the wrong entry shows."""
    page_bytes = b.page_size * b.row_bytes
    owner = torch.from_numpy(np.arange(b.n_pool_pages) % b.n_pool_entries).cuda()
    arenas = []
    for e in range(b.n_pool_entries):
        a = pool.clone().view(b.n_pool_pages, page_bytes)
        a[owner != e] = POISON
        arenas.append(a.view(-1))
    return arenas


@pytest.mark.parametrize("which", ["full_table", "multi_source"])
def test_pool_entries_as_distinct_owner_arenas(orc, which):
    """The pool entries of the table are distinct arenas, each holding only
    the pages its entry owns (page mod NP), the rest poisoned: the one-launch
    layer, the two-launch layer and the record split read every prefix page
    from its owner's arena and match the oracle (which reads one pool)."""
    gpb = _gpb()
    b = _full_table_batch() if which == "full_table" else workloads.make_batch(which)
    if which == "full_table":
        pool_np, cur_np = pins.tagged_values(b)
        pools, curs = [torch.from_numpy(pool_np).cuda()], [torch.from_numpy(cur_np).cuda()]
    else:
        pools, curs = workloads.make_values(b, device="cuda")
        pool_np, cur_np = _host(pools[0]), _host(curs[0])
    r = _runner(b, pools, curs)
    r.begin_batch()
    torch.cuda.synchronize()
    want_plan = _check_plan(b, r, orc)
    want, want_staging = _oracle_layer(b, want_plan, pool_np, cur_np, orc)
    arenas = _owner_arenas(b, pools[0])
    slab = b.staging_cap_pages * b.page_size * b.row_bytes
    base = r.staging[0].data_ptr()
    table = gpb.Sources([(a, b.n_pool_pages) for a in arenas] +
                        [(base + w * slab, b.staging_cap_pages) for w in range(b.n_writers)])
    NCP = r.plan.NCP
    runs = {
        "one launch": lambda: gpb.compose_layer(
            r.dense[0], table, r.plan, r.S, NCP, r.staging[0], r.staging_rows_total, curs[0],
            r.T, r.ps, r.rb, r.status),
        "two launches": lambda: (
            gpb.current_row_scatter(r.staging[0], r.staging_rows_total,
                                    r.plan.t["staging_rows"], curs[0], r.T, r.rb, r.status),
            gpb.compose_gather(r.dense[0], table, r.plan.t["owner"], r.plan.t["src"], r.S,
                               r.ps, r.rb, r.status)),
        "record split": lambda: (
            gpb.compose_gather_records(r.dense[0], table, r.plan.t["prefix_desc"],
                                       r.S - NCP, r.S, r.ps, r.rb, r.status),
            gpb.compose_consume(r.dense[0], table, r.plan, r.S, NCP, r.staging[0],
                                r.staging_rows_total, curs[0], r.T, r.ps, r.rb, r.status)),
    }
    for what, run in runs.items():
        _say(which, what, "NP", b.n_pool_entries, "W", b.n_writers)
        r.dense[0].fill_(POISON)
        run()
        torch.cuda.synchronize()
        got = _host(r.dense_of(0))
        if not np.array_equal(got, want):
            bad_rows = np.nonzero((got != want).any(axis=1))[0]
            raise AssertionError("%s, %s: %d dense rows differ, first %s"
                                 % (which, what, len(bad_rows), bad_rows[:8].tolist()))
        assert np.array_equal(_host(r.staging_of(0)), want_staging), what
        assert _status(r) == 0, what


def test_empty_and_degenerate_batches(orc):
    cases = [([], []), ([0, 0], [0, 0]), ([3, 2], [0, 0]), ([0, 0], [5, 64]),
             ([1], [65])]
    for P, c in cases:
        P = np.array(P, np.int32)
        c = np.array(c, np.int32)
        n = int(P.sum() + ((c + 63) // 64).sum())
        pages = np.arange(2, n + 2, dtype=np.int32)
        b = workloads.Batch("edge", len(P), 64, 64, n + 3, 1, 1,
                            workloads.staging_cap_for(int(c.sum()), len(P)), P, c, pages)
        _random_case(orc, b)


def test_sentinel_and_out_of_range_descriptors(orc):
    """-1 descriptors zero-fill (page d63fbd4, commit "compose_v2"); a
    descriptor outside the table or its arena is zero-filled and flagged."""
    gpb = _gpb()
    PS, RB = 4, 64
    rng = np.random.default_rng(11)
    pool_np = rng.integers(1, 256, (10 * PS, RB), dtype=np.uint8)
    stag_np = rng.integers(1, 256, (3 * PS, RB), dtype=np.uint8)
    pool = torch.from_numpy(pool_np).cuda()
    stag = torch.from_numpy(stag_np).cuda()
    owner = np.array([-1, 0, 1, 0, 2, 0, 1, -1], np.int32)
    src = np.array([4, -1, 2, 9, 0, 10, 3, -1], np.int32)
    dense = torch.full((len(owner) * PS, RB), 0x77, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpb.compose_gather(dense, [(pool, 10), (stag, 3)], torch.from_numpy(owner).cuda(),
                       torch.from_numpy(src).cuda(), len(owner), PS, RB, status)
    torch.cuda.synchronize()
    table = [pool_np.reshape(-1), stag_np.reshape(-1)]
    want, bad = orc.compose_layer(table, np.zeros((0, RB), np.uint8), np.zeros(0, np.int32),
                                  owner, src, PS, RB, np.zeros(RB, np.uint8))
    assert bad
    assert np.array_equal(_host(dense), want)
    assert int(status.item()) == gpb.STATUS_BAD_DESCRIPTOR


def test_plan_reports_device_metadata_that_differs_from_the_host(orc):
    """The host validates its own copies of the metadata; if the device copies
    say something else (page ids out of range, a longer prefix), the plan
    kernels keep every write inside its array and set the plan status bit.
    A later plan from consistent copies is exact again."""
    gpb = _gpb()
    b = workloads.make_batch("medium")
    meta = gpb.BatchMeta.of(b)
    p = gpb.Plan(meta)
    bad = p.d_req.clone()
    bad[0] = b.n_pool_pages + 5
    bad[7] = -3
    p.d_req.copy_(bad)
    p.build()
    torch.cuda.synchronize()
    assert int(p.status.item()) & gpb.STATUS_BAD_PLAN_INPUT
    p.d_req.copy_(torch.from_numpy(meta.h_req).cuda())
    p.d_prefix.copy_(p.d_prefix + 3)
    p.status.zero_()
    p.build()
    torch.cuda.synchronize()
    assert int(p.status.item()) & gpb.STATUS_BAD_PLAN_INPUT
    p.d_prefix.copy_(torch.from_numpy(meta.h_prefix).cuda())
    p.status.zero_()
    p.build()
    torch.cuda.synchronize()
    assert int(p.status.item()) == 0
    want = oracle.plan_for(b, orc)
    for k in oracle.PLAN_FIELDS:
        assert np.array_equal(_host(p.t[k]), want[k]), k


def test_slot_list_out_of_range_is_skipped(orc):
    """A listed slot outside the dense buffer is skipped and flagged; the
    others are gathered."""
    gpb = _gpb()
    PS, RB = 2, 32
    rng = np.random.default_rng(13)
    pool_np = rng.integers(1, 256, (6 * PS, RB), dtype=np.uint8)
    pool = torch.from_numpy(pool_np).cuda()
    owner = torch.zeros(4, dtype=torch.int32, device="cuda")
    src = torch.tensor([1, 2, 3, 4], dtype=torch.int32, device="cuda")
    dense = torch.full((4 * PS, RB), 0x33, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    slots = torch.tensor([2, 9, -1, 0], dtype=torch.int32, device="cuda")
    gpb.compose_gather_slots(dense, [(pool, 6)], slots, 4, owner, src, 4, PS, RB, status)
    torch.cuda.synchronize()
    h = _host(dense).reshape(4, PS, RB)
    want = np.full((4, PS, RB), 0x33, np.uint8)
    want[2] = pool_np[3 * PS:4 * PS]
    want[0] = pool_np[1 * PS:2 * PS]
    assert np.array_equal(h, want)
    assert int(status.item()) == gpb.STATUS_BAD_DESCRIPTOR


def test_out_of_range_staging_rows_are_skipped(orc):
    gpb = _gpb()
    RB = 32
    rng = np.random.default_rng(12)
    cur_np = rng.integers(1, 256, (5, RB), dtype=np.uint8)
    rows = np.array([3, -1, 7, 8, 0], np.int32)        # 8 rows of staging: 8 is out
    stag = torch.zeros((8, RB), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpb.current_row_scatter(stag, 8, torch.from_numpy(rows).cuda(),
                            torch.from_numpy(cur_np).cuda(), 5, RB, status)
    torch.cuda.synchronize()
    want = np.zeros((8, RB), np.uint8)
    want[3], want[7], want[0] = cur_np[0], cur_np[2], cur_np[4]
    assert np.array_equal(_host(stag), want)
    assert int(status.item()) == gpb.STATUS_BAD_STAGING_ROW


@pytest.mark.parametrize("start,n", [(16, 4096 * 37), (16, 16), (48, 4096 * 37 + 16 * 5),
                                     (0, 4080), (4096, 4112), (32, 3 * 4096 - 16)])
def test_staging_clear_zeroes_exactly(orc, start, n):
    """Exactly [start, start + n) becomes zero, including a last workgroup
    that covers less than its 4 KiB."""
    gpb = _gpb()
    buf = torch.full((1 << 20,), 0xEE, dtype=torch.uint8, device="cuda")
    gpb.staging_clear(buf[start:start + n], n)
    torch.cuda.synchronize()
    h = _host(buf)
    assert not h[start:start + n].any()
    assert (h[:start] == 0xEE).all() and (h[start + n:] == 0xEE).all()


def test_index_key_twin_shares_the_plan(orc):
    """The indexer-key twin (page 0d87bc5, commit "prefetch staging exchange":
    the index fill is pointed at the same staging page inverse) composes a
    second row format with the token plan of the traced batch: 144-byte rows,
    byte-exact against the oracle on four layers, each with its own pool and
    current-row arena and with both formats' dense halves poisoned first."""
    gpb = _gpb()
    b = workloads.make_batch("traced")
    rb = workloads.INDEX_ROW_BYTES
    pools, curs = workloads.make_values(b, device="cuda", rotations=4)
    tok = _runner(b, pools, curs)
    ipools, icurs = workloads.make_values(b, device="cuda", rotations=4, row_bytes=rb,
                                          value_kind="bytes", seed=1)
    twin = gpb.ComposeRunner(gpb.BatchMeta(b.bs, b.page_size, rb, b.n_pool_pages,
                                           b.n_pool_entries, b.n_writers,
                                           b.staging_cap_pages, b.prefix_pages,
                                           b.cur_tokens, b.req_pages),
                             ipools, icurs, plan=tok.plan)
    tok.begin_batch()
    twin.begin_batch()
    bi = workloads.Batch(b.name, b.bs, b.page_size, rb, b.n_pool_pages, b.n_pool_entries,
                         b.n_writers, b.staging_cap_pages, b.prefix_pages, b.cur_tokens,
                         b.req_pages)
    want = oracle.plan_for(bi, orc)
    ipools_np = [_host(p) for p in ipools]
    icurs_np = [_host(c) for c in icurs]
    pools_np, curs_np = [_host(p) for p in pools], [_host(c) for c in curs]
    for layer in range(4):
        # a page either format fails to write shows against the sentinel,
        # not against what layer - 2 left in the same half
        tok.dense[layer % 2].fill_(POISON)
        twin.dense[layer % 2].fill_(POISON)
        tok.layer(layer)
        twin.layer(layer)
        torch.cuda.synchronize()
        _check_layer(bi, twin, layer, want, ipools_np, icurs_np, orc)
        _check_layer(b, tok, layer, want, pools_np, curs_np, orc, check_staging=False)
        _say("  twin layer", layer, "ok")
    assert _status(twin) == 0 and _status(tok) == 0


def test_batch_replays_in_a_hip_graph(orc):
    """The whole batch (plan build, staging clears, two layers of scatter and
    gather) captured in a HIP graph on a side stream: every replay, with
    eager work that dirties the outputs in between, reproduces the eager
    result, which matches the oracle.  The staging clear is a kernel, so the
    graph holds no memset node."""
    b = workloads.make_batch("medium")
    pools, curs = workloads.make_values(b, device="cuda", rotations=2)
    r = _runner(b, pools, curs)
    r.run(2)
    torch.cuda.synchronize()
    want = _check_plan(b, r, orc)
    pools_np = [_host(p) for p in pools]
    curs_np = [_host(c) for c in curs]
    for layer in (0, 1):
        _check_layer(b, r, layer, want, pools_np, curs_np, orc)
    ref = [t.clone() for t in r.dense + r.staging]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        r.run(2, side)
    for rep in range(3):
        for k, t in enumerate(r.dense + r.staging):
            t.fill_(0x11 * (k + 1))
        for k in r.plan.t:
            r.plan.t[k].fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b_ in zip(r.dense + r.staging, ref):
            assert torch.equal(a, b_), "replay %d differs from the eager run" % rep
        for k in oracle.PLAN_FIELDS:
            assert np.array_equal(_host(r.plan.t[k]), want[k]), (rep, k)
        _say("  replay", rep, "ok")
    assert _status(r) == 0


@pytest.mark.parametrize("schedule", ["one_stream", "two_streams"])
def test_layer_ahead_schedule_replays_in_a_hip_graph(orc, schedule):
    """The layer-ahead schedules (one launch per layer on one stream; prefix
    gathers on a second stream ordered by events) over four layers of the
    medium batch with four arenas, captured once in a HIP graph: every
    replay, with eager work that dirties every output in between, gives the
    eager run's dense halves, staging and plan, and the last two layers match
    the oracle."""
    b = workloads.make_batch("medium")
    L = 4
    pools, curs = workloads.make_values(b, device="cuda", rotations=L)
    r = _runner(b, pools, curs)
    main = torch.cuda.current_stream()

    def schedule_on(stream, side):
        if schedule == "one_stream":
            r.run_layer_ahead(L, stream)
        else:
            r.run_pipelined(L, stream, side, consume="fused")

    schedule_on(main, torch.cuda.Stream())
    torch.cuda.synchronize()
    want = _check_plan(b, r, orc)
    pools_np = [_host(p) for p in pools]
    curs_np = [_host(c) for c in curs]
    for layer in (L - 2, L - 1):
        _check_layer(b, r, layer, want, pools_np, curs_np, orc)
    ref = [t.clone() for t in r.dense + r.staging]
    cap = torch.cuda.Stream()
    cap.wait_stream(main)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        schedule_on(cap, side)
    for rep in range(3):
        for k, t in enumerate(r.dense + r.staging):
            t.fill_(0x11 * (k + 1))
        for k in r.plan.t:
            r.plan.t[k].fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b_ in zip(r.dense + r.staging, ref):
            assert torch.equal(a, b_), "replay %d differs from the eager run" % rep
        for k in oracle.PLAN_FIELDS:
            assert np.array_equal(_host(r.plan.t[k]), want[k]), (rep, k)
        _say("  replay", rep, schedule, "ok")
    assert _status(r) == 0


@pytest.mark.parametrize("seed", range(2))
def test_grouped_formats_match_single_format(orc, seed):
    """Two to four row formats (four, the most a launch takes, on the first
    batch) on one plan, composed with one launch per layer for all of them
    and with one scatter launch and one gather launch for all of them, give
    per format the single-format result (the oracle's)."""
    gpb = _gpb()
    rng = np.random.default_rng(900 + seed)
    for i in range(12):
        b = workloads.random_batch(rng, page_size=int(rng.choice([1, 4, 16, 64])))
        extra = 3 if i == 0 else int(rng.integers(1, 4))
        sizes = [b.row_bytes] + [int(16 * rng.integers(1, 10)) for _ in range(extra)]
        runners, host = [], []
        plan = None
        for k, rb in enumerate(sizes):
            bk = workloads.Batch(b.name, b.bs, b.page_size, rb, b.n_pool_pages,
                                 b.n_pool_entries, b.n_writers, b.staging_cap_pages,
                                 b.prefix_pages, b.cur_tokens, b.req_pages)
            pool_np, cur_np = pins.tagged_values(bk, seed=seed * 100 + i * 10 + k)
            meta = gpb.BatchMeta.of(bk)
            r = gpb.ComposeRunner(meta, [torch.from_numpy(pool_np).cuda()],
                                  [torch.from_numpy(cur_np).cuda()], plan=plan)
            plan = r.plan
            runners.append(r)
            host.append((bk, pool_np, cur_np))
        for grouped in (gpb.layer_groups, gpb.layer_groups_two_launch):
            for r in runners:
                r.begin_batch()
                for d in r.dense:
                    d.fill_(POISON)
            for layer in range(2):
                grouped(runners, layer)
            torch.cuda.synchronize()
            want = _check_plan(host[0][0], runners[0], orc)
            for r, (bk, pool_np, cur_np) in zip(runners, host):
                for layer in range(2):
                    _check_layer(bk, r, layer, want, [pool_np], [cur_np], orc)
                assert _status(r) == 0
    _say("grouped seed", seed, "ok")


def test_token_and_index_twin_in_one_launch_each(orc):
    """The traced batch's token KV (1152-byte rows) and index keys (144-byte
    rows) composed with grouped launches (one per layer, and scatter + gather),
    four layers each with distinct arenas and poisoned dense halves,
    byte-exact."""
    gpb = _gpb()
    b = workloads.make_batch("traced")
    rb = workloads.INDEX_ROW_BYTES
    pools, curs = workloads.make_values(b, device="cuda", rotations=4)
    tok = _runner(b, pools, curs)
    ipools, icurs = workloads.make_values(b, device="cuda", rotations=4, row_bytes=rb,
                                          value_kind="bytes", seed=1)
    bi = workloads.Batch(b.name, b.bs, b.page_size, rb, b.n_pool_pages, b.n_pool_entries,
                         b.n_writers, b.staging_cap_pages, b.prefix_pages, b.cur_tokens,
                         b.req_pages)
    twin = gpb.ComposeRunner(gpb.BatchMeta.of(bi), ipools, icurs, plan=tok.plan)
    tok.begin_batch()
    twin.begin_batch()
    want = _check_plan(b, tok, orc)
    pools_np, curs_np = [_host(p) for p in pools], [_host(c) for c in curs]
    ipools_np, icurs_np = [_host(p) for p in ipools], [_host(c) for c in icurs]
    for grouped in (gpb.layer_groups, gpb.layer_groups_two_launch):
        for layer in range(4):
            tok.dense[layer % 2].fill_(POISON)
            twin.dense[layer % 2].fill_(POISON)
            grouped([tok, twin], layer)
            torch.cuda.synchronize()
            _check_layer(b, tok, layer, want, pools_np, curs_np, orc)
            _check_layer(bi, twin, layer, want, ipools_np, icurs_np, orc)
            _say("  grouped layer", layer, grouped.__name__, "ok")
    assert _status(tok) == 0 and _status(twin) == 0
