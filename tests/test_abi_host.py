"""CPU-only checks of the C ABI: the library loads, exports every function
include/gpb.h declares, and rejects bad arguments on the host before any
launch (page d63fbd4, commit "touched-pages-proportional staging": overflow
fails fast; page 0d87bc5, commit "prefetch staging exchange": page 0 is the
dummy page).  No call here reaches a kernel launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import gather_plan_build_amd as gpb
from gather_plan_build_amd import binding as B
import oracle
import pins
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "gpb.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(gpb_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    assert header_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(gpb.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_strerror_names_every_status():
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert gpb.strerror(code) and "unknown" not in gpb.strerror(code)
    assert "unknown" in gpb.strerror(-99)


def _meta(**kw):
    base = dict(bs=2, page_size=64, row_bytes=1152, n_pool_pages=16, n_pool_entries=1,
                n_writers=1, staging_cap_pages=4, prefix_pages=[1, 1], cur_tokens=[64, 65],
                req_pages=[1, 2, 3, 4, 5])
    base.update(kw)
    return B.BatchMeta(**base)


@pytest.mark.parametrize("kw,code", [
    ({}, B.OK),
    (dict(req_pages=[0, 2, 3, 4, 5]), B.EPAGE),          # dummy page 0
    (dict(req_pages=[1, 2, 3, 4, 1]), B.EPAGE),          # repeated page
    (dict(req_pages=[1, 2, 3, 4, 16]), B.EPAGE),         # beyond the pool
    (dict(req_pages=[1, 2, 3, 4, -2]), B.EPAGE),
    (dict(staging_cap_pages=3), B.ECAPACITY),            # slot 0 + 3 pages
    (dict(row_bytes=1000), B.EALIGN),
    (dict(row_bytes=0), B.EINVAL),
    (dict(page_size=0), B.EINVAL),
    (dict(n_writers=0), B.EINVAL),
    (dict(n_pool_entries=0), B.EINVAL),
    (dict(prefix_pages=[1, -1]), B.EINVAL),
    (dict(cur_tokens=[64, -3]), B.EINVAL),
    (dict(bs=-1), B.EINVAL),
    (dict(page_size=1 << 20, n_pool_pages=4096), B.ERANGE),
])
def test_plan_sizes_validation(kw, code):
    m = _meta(**kw)
    rc = B.lib.gpb_plan_sizes(ctypes.byref(m.c), None, None, None)
    assert rc == code, gpb.strerror(rc)


def test_empty_batch_is_valid():
    m = B.BatchMeta(0, 64, 16, 8, 1, 1, 1, [], [], [])
    assert gpb.plan_sizes(m) == (0, 0, 0)


def test_plan_build_rejects_before_launch():
    m = _meta(req_pages=[0, 2, 3, 4, 5])
    p = B.gpb_plan()
    assert B.lib.gpb_plan_build(ctypes.byref(m.c), ctypes.byref(p), None) == B.EPAGE
    ok = _meta()
    # valid batch but no device arrays / outputs: rejected on the host
    assert B.lib.gpb_plan_build(ctypes.byref(ok.c), ctypes.byref(p), None) == B.EINVAL
    assert B.lib.gpb_plan_build(ctypes.byref(ok.c), None, None) == B.EINVAL
    assert B.lib.gpb_plan_build(None, ctypes.byref(p), None) == B.EINVAL


def test_plan_build_rejects_misaligned_outputs():
    m = _meta()
    fake = 0x100000  # never dereferenced: the check fails before any launch
    m.c.d_prefix_pages = fake
    m.c.d_cur_tokens = fake
    m.c.d_req_pages = fake
    p = B.gpb_plan(*([fake] * len(B.PLAN_FIELDS)))
    p.d_owner = fake + 2
    assert B.lib.gpb_plan_build(ctypes.byref(m.c), ctypes.byref(p), None) == B.EALIGN


def test_scatter_argument_checks():
    f = B.lib.gpb_current_row_scatter
    a = 0x100000
    assert f(a, 10, a, a, 0, 1152, None, None) == B.OK          # empty: no launch
    assert f(a, 10, a, a, -1, 1152, None, None) == B.EINVAL
    assert f(a, 10, a, a, 4, 1000, None, None) == B.EALIGN
    assert f(a + 8, 10, a, a, 4, 1152, None, None) == B.EALIGN
    assert f(a, 10, a + 2, a, 4, 1152, None, None) == B.EALIGN
    assert f(None, 10, a, a, 4, 1152, None, None) == B.EINVAL
    assert f(a, 1 << 40, a, a, 4, 1152, None, None) == B.ERANGE
    assert f(a, 10, a, a, 1 << 22, 1152, None, None) == B.ERANGE   # > 2 GiB of rows


def test_gather_argument_checks():
    f = B.lib.gpb_compose_gather
    a = 0x100000
    good = B.Sources([(a, 10), (a, 4)])
    assert f(a, ctypes.byref(good.c), a, a, 0, 64, 1152, None, None) == B.OK  # no slots
    assert f(a, None, a, a, 4, 64, 1152, None, None) == B.EINVAL
    assert f(a, ctypes.byref(good.c), a, a, -1, 64, 1152, None, None) == B.EINVAL
    assert f(a, ctypes.byref(good.c), a, a, 4, 0, 1152, None, None) == B.EINVAL
    assert f(a, ctypes.byref(good.c), a, a, 4, 64, 1000, None, None) == B.EALIGN
    assert f(a + 4, ctypes.byref(good.c), a, a, 4, 64, 1152, None, None) == B.EALIGN
    assert f(None, ctypes.byref(good.c), a, a, 4, 64, 1152, None, None) == B.EINVAL
    bad = B.Sources([(a + 8, 10)])
    assert f(a, ctypes.byref(bad.c), a, a, 4, 64, 1152, None, None) == B.EALIGN
    neg = B.Sources([(a, -1)])
    assert f(a, ctypes.byref(neg.c), a, a, 4, 64, 1152, None, None) == B.EINVAL
    empty = B.gpb_sources()
    assert f(a, ctypes.byref(empty), a, a, 4, 64, 1152, None, None) == B.EINVAL
    assert f(a, ctypes.byref(good.c), a, a, 4, 1 << 20, 4096, None, None) == B.ERANGE
    # the table holds at most GPB_MAX_SOURCES entries
    full = B.Sources([(a, 10)] * B.MAX_SOURCES)
    assert f(a, ctypes.byref(full.c), a, a, 0, 64, 1152, None, None) == B.OK
    over = B.gpb_sources()
    over.n = B.MAX_SOURCES + 1
    assert f(a, ctypes.byref(over), a, a, 4, 64, 1152, None, None) == B.EINVAL
    with pytest.raises(B.GpbError):
        B.Sources([(a, 10)] * (B.MAX_SOURCES + 1))


def test_slot_gather_and_fill_argument_checks():
    g = B.lib.gpb_compose_gather_slots
    a = 0x100000
    good = B.Sources([(a, 10)])
    assert g(a, ctypes.byref(good.c), a, 0, a, a, 4, 64, 1152, None, None) == B.OK
    assert g(a, ctypes.byref(good.c), a, -1, a, a, 4, 64, 1152, None, None) == B.EINVAL
    assert g(a, ctypes.byref(good.c), None, 3, a, a, 4, 64, 1152, None, None) == B.EINVAL
    assert g(a, ctypes.byref(good.c), a + 2, 3, a, a, 4, 64, 1152, None, None) == B.EALIGN
    assert g(a, ctypes.byref(good.c), a, 3, a, a, 0, 64, 1152, None, None) == B.EINVAL
    assert g(a, None, a, 3, a, a, 4, 64, 1152, None, None) == B.EINVAL
    f = B.lib.gpb_current_row_fill
    assert f(a, 10, a, a, 100, a, a, 0, 1152, None, None) == B.OK
    assert f(a, 10, a, None, 100, a, a, 4, 1152, None, None) == B.EINVAL
    assert f(a, 10, a, a, -1, a, a, 4, 1152, None, None) == B.EINVAL
    assert f(a, 10, a, a + 8, 100, a, a, 4, 1152, None, None) == B.EALIGN
    assert f(a, 10, a, a, 100, a + 1, a, 4, 1152, None, None) == B.EALIGN
    assert f(a, 10, a, a, 100, a, a, 4, 1000, None, None) == B.EALIGN


def test_record_gather_argument_checks():
    g = B.lib.gpb_compose_gather_records
    a = 0x100000
    good = B.Sources([(a, 10)])
    assert g(a, ctypes.byref(good.c), a, 0, 4, 64, 1152, None, None) == B.OK
    assert g(a, ctypes.byref(good.c), a, -1, 4, 64, 1152, None, None) == B.EINVAL
    assert g(a, ctypes.byref(good.c), None, 3, 4, 64, 1152, None, None) == B.EINVAL
    assert g(a, ctypes.byref(good.c), a + 4, 3, 4, 64, 1152, None, None) == B.EALIGN
    assert g(a + 4, ctypes.byref(good.c), a, 3, 4, 64, 1152, None, None) == B.EALIGN
    assert g(a, ctypes.byref(good.c), a, 3, 0, 64, 1152, None, None) == B.EINVAL
    assert g(a, None, a, 3, 4, 64, 1152, None, None) == B.EINVAL


def test_one_launch_layer_argument_checks():
    a = 0x100000
    good = B.Sources([(a, 10), (a, 4)])
    p = B.gpb_plan(*([a] * len(B.PLAN_FIELDS)))
    ahead = B.lib.gpb_compose_layer_ahead
    # the next layer's dense buffer is required (with prefix pages) and aligned
    assert ahead(a, None, ctypes.byref(good.c), ctypes.byref(p), 4, 1, a, 10, a, 5, 64, 1152,
                 None, None) == B.EINVAL
    assert ahead(a, a + 8, ctypes.byref(good.c), ctypes.byref(p), 4, 1, a, 10, a, 5, 64,
                 1152, None, None) == B.EALIGN
    for f in (B.lib.gpb_compose_layer, B.lib.gpb_compose_consume,
              lambda *x: ahead(x[0], a, *x[1:])):
        # dense, table, plan, S, NCP, staging, staging rows, cur, T, PS, RB
        assert f(a, ctypes.byref(good.c), ctypes.byref(p), 0, 0, a, 10, a, 0, 64, 1152,
                 None, None) == B.OK
        assert f(a, ctypes.byref(good.c), None, 4, 1, a, 10, a, 5, 64, 1152,
                 None, None) == B.EINVAL
        assert f(a, ctypes.byref(good.c), ctypes.byref(p), 4, 5, a, 10, a, 5, 64, 1152,
                 None, None) == B.EINVAL                       # NCP > S
        assert f(a, ctypes.byref(good.c), ctypes.byref(p), 4, 2, a, 10, a, 1, 64, 1152,
                 None, None) == B.EINVAL                       # NCP > T
        assert f(a, ctypes.byref(good.c), ctypes.byref(p), 4, 1, None, 10, a, 5, 64, 1152,
                 None, None) == B.EINVAL
        assert f(a, ctypes.byref(good.c), ctypes.byref(p), 4, 1, a + 8, 10, a, 5, 64, 1152,
                 None, None) == B.EALIGN
        assert f(a, ctypes.byref(good.c), ctypes.byref(p), 4, 1, a, 1 << 40, a, 5, 64,
                 1152, None, None) == B.ERANGE
        assert f(a, ctypes.byref(good.c), ctypes.byref(p), 4, 1, a, 10, a, 1 << 22, 64,
                 1152, None, None) == B.ERANGE               # > 2 GiB of rows
        q = B.gpb_plan(*([a] * len(B.PLAN_FIELDS)))
        q.d_current_desc = a + 4
        assert f(a, ctypes.byref(good.c), ctypes.byref(q), 4, 1, a, 10, a, 5, 64, 1152,
                 None, None) == B.EALIGN
        q.d_current_desc = None
        assert f(a, ctypes.byref(good.c), ctypes.byref(q), 4, 1, a, 10, a, 5, 64, 1152,
                 None, None) == B.EINVAL


def test_noalloc_layer_argument_checks():
    """Everything the static-staging layer can refuse without a device is
    refused on the host: the table of pool entries, the writer count, the row
    size and staging beyond GPB_SCRATCH_BYTES (GPB_ESCRATCH)."""
    a = 0x100000
    f = B.lib.gpb_compose_layer_noalloc
    p = B.gpb_plan(*([a] * len(B.PLAN_FIELDS)))
    pools = B.Sources([(a, 10)])
    full = B.Sources([(a, 10)] * B.MAX_SOURCES)

    def call(pool_table, W, CAP, PS=64, RB=1152):
        # dense, pools, W, CAP, plan, S, NCP, cur, T, PS, RB, status, stream
        return f(a, None if pool_table is None else ctypes.byref(pool_table.c), W, CAP,
                 ctypes.byref(p), 4, 1, a, 5, PS, RB, None, None)

    assert call(None, 1, 4) == B.EINVAL
    assert call(pools, 0, 4) == B.EINVAL                       # no writer
    assert call(pools, 1, 0) == B.EINVAL                       # no staging page
    assert call(full, 1, 4) == B.EINVAL                        # 64 pools + 1 slab
    assert call(B.Sources([(a, 10)] * 60), 5, 4) == B.EINVAL
    assert call(pools, 1, 4, PS=0) == B.EINVAL
    assert call(pools, 1, 4, RB=1000) == B.EALIGN
    rows_max = B.SCRATCH_BYTES // 1152
    assert call(pools, 1, rows_max // 64 + 1) == B.ESCRATCH     # one slab too large
    assert call(pools, 8, rows_max // 64 // 8 + 1) == B.ESCRATCH
    assert call(pools, 1, 1 << 30, PS=1 << 30, RB=16) == B.ESCRATCH  # no overflow
    assert call(pools, 63, (1 << 31) - 1, PS=(1 << 31) - 1, RB=16) == B.ESCRATCH
    assert "scratch" in gpb.strerror(B.ESCRATCH)


def test_layer_groups_argument_checks():
    f = B.lib.gpb_compose_layer_groups
    a = 0x100000
    t = B.Sources([(a, 10), (a, 4)])
    p = B.gpb_plan(*([a] * len(B.PLAN_FIELDS)))

    def groups(*gs):
        return (B.gpb_layer_group * len(gs))(*gs)

    good = B.gpb_layer_group(a, ctypes.pointer(t.c), a, 10, a, 1152)
    # groups, n, plan, S, NCP, T, PS
    assert f(groups(good), 1, ctypes.byref(p), 0, 0, 0, 64, None, None) == B.OK
    assert f(groups(good), 0, ctypes.byref(p), 4, 1, 5, 64, None, None) == B.EINVAL
    assert f(groups(good), B.MAX_GROUPS + 1, ctypes.byref(p), 4, 1, 5, 64, None,
             None) == B.EINVAL
    assert f(groups(good), 1, None, 4, 1, 5, 64, None, None) == B.EINVAL
    assert f(groups(good), 1, ctypes.byref(p), 4, 2, 1, 64, None, None) == B.EINVAL
    big = B.Sources([(a, 10)] * (B.MAX_GROUP_SOURCES + 1))
    over = B.gpb_layer_group(a, ctypes.pointer(big.c), a, 10, a, 1152)
    assert f(groups(over), 1, ctypes.byref(p), 4, 1, 5, 64, None, None) == B.EINVAL
    odd = B.gpb_layer_group(a, ctypes.pointer(t.c), a, 10, a, 1000)
    assert f(groups(odd), 1, ctypes.byref(p), 4, 1, 5, 64, None, None) == B.EALIGN
    mis = B.gpb_layer_group(a, ctypes.pointer(t.c), a + 8, 10, a, 1152)
    assert f(groups(good, mis), 2, ctypes.byref(p), 4, 1, 5, 64, None, None) == B.EALIGN
    nost = B.gpb_layer_group(a, ctypes.pointer(t.c), None, 10, a, 1152)
    assert f(groups(nost), 1, ctypes.byref(p), 4, 1, 5, 64, None, None) == B.EINVAL
    q = B.gpb_plan(*([a] * len(B.PLAN_FIELDS)))
    q.d_prefix_desc = a + 4
    assert f(groups(good), 1, ctypes.byref(q), 4, 1, 5, 64, None, None) == B.EALIGN


@pytest.mark.parametrize("which", ["layer_fill", "consume_fill", "ahead_fill"])
def test_layer_fill_argument_checks(which):
    a = 0x100000
    if which == "ahead_fill":
        def f(*x):
            return B.lib.gpb_compose_layer_ahead_fill(x[0], a, *x[1:])
    else:
        f = getattr(B.lib, "gpb_compose_" + which)
    t = B.Sources([(a, 10), (a, 4)])
    p = B.gpb_plan(*([a] * len(B.PLAN_FIELDS)))
    # dense, table, plan, S, NCP, staging, staging rows, pool, pool rows, cur, T, PS, RB
    assert f(a, ctypes.byref(t.c), ctypes.byref(p), 0, 0, a, 10, a, 100, a, 0, 64, 1152,
             None, None) == B.OK
    assert f(a, ctypes.byref(t.c), ctypes.byref(p), 4, 1, a, 10, a, -1, a, 5, 64, 1152,
             None, None) == B.EINVAL
    assert f(a, ctypes.byref(t.c), ctypes.byref(p), 4, 1, a, 10, None, 100, a, 5, 64, 1152,
             None, None) == B.EINVAL
    assert f(a, ctypes.byref(t.c), ctypes.byref(p), 4, 1, a, 10, a + 8, 100, a, 5, 64, 1152,
             None, None) == B.EALIGN
    q = B.gpb_plan(*([a] * len(B.PLAN_FIELDS)))
    q.d_pool_locs = None
    assert f(a, ctypes.byref(t.c), ctypes.byref(q), 4, 1, a, 10, a, 100, a, 5, 64, 1152,
             None, None) == B.EINVAL
    assert f(a, ctypes.byref(t.c), None, 4, 1, a, 10, a, 100, a, 5, 64, 1152,
             None, None) == B.EINVAL
    if which == "ahead_fill":
        # the next layer's dense buffer is required (with prefix pages) and aligned
        g = B.lib.gpb_compose_layer_ahead_fill
        assert g(a, None, ctypes.byref(t.c), ctypes.byref(p), 4, 1, a, 10, a, 100, a, 5, 64,
                 1152, None, None) == B.EINVAL
        assert g(a, a + 8, ctypes.byref(t.c), ctypes.byref(p), 4, 1, a, 10, a, 100, a, 5, 64,
                 1152, None, None) == B.EALIGN


def test_plan_build_clear_and_writer_counts_checks():
    m = _meta()
    fake = 0x100000
    m.c.d_prefix_pages = fake
    m.c.d_cur_tokens = fake
    m.c.d_req_pages = fake
    p = B.gpb_plan(*([fake] * len(B.PLAN_FIELDS)))
    f = B.lib.gpb_plan_build_clear
    assert f(ctypes.byref(m.c), ctypes.byref(p), None, 64, None) == B.EINVAL
    assert f(ctypes.byref(m.c), ctypes.byref(p), fake, -16, None) == B.EINVAL
    assert f(ctypes.byref(m.c), ctypes.byref(p), fake + 8, 64, None) == B.EALIGN
    assert f(ctypes.byref(m.c), ctypes.byref(p), fake, 40, None) == B.EALIGN
    p.d_prefix_desc = fake + 4   # records are 16-byte aligned
    assert B.lib.gpb_plan_build(ctypes.byref(m.c), ctypes.byref(p), None) == B.EALIGN
    # per-writer list sizes on the host: 2 writers, current pages of 64 and
    # 65 tokens -> pages (64 | 64, 1) dealt 0, 1, 0
    w = _meta(n_writers=2, staging_cap_pages=4)
    counts = np.zeros(2, np.int32)
    assert B.lib.gpb_writer_counts(ctypes.byref(w.c),
                                   counts.ctypes.data_as(B._I32P)) == B.OK
    assert counts.tolist() == [64 + 1, 64]
    assert B.lib.gpb_writer_counts(ctypes.byref(w.c), None) == B.EINVAL
    bad = _meta(req_pages=[0, 2, 3, 4, 5])
    assert B.lib.gpb_writer_counts(ctypes.byref(bad.c),
                                   counts.ctypes.data_as(B._I32P)) == B.EPAGE


def test_writer_counts_agree_with_oracle(orc):
    """The host-side list sizes equal the differences of the oracle's
    writer_offsets on random multi-writer batches."""
    for b in pins.random_batches(40, seed=77, n_writers=5, n_pool_entries=2):
        want = np.diff(oracle.plan_for(b, orc)["writer_offsets"])
        assert np.array_equal(gpb.writer_counts(gpb.BatchMeta.of(b)), want)


def test_group_argument_checks():
    a = 0x100000
    t = B.Sources([(a, 10), (a, 4)])
    big = B.Sources([(a, 1)] * 17)

    def gg(*groups):
        return (B.gpb_gather_group * len(groups))(*groups)

    def rg(*groups):
        return (B.gpb_row_group * len(groups))(*groups)

    G = B.lib.gpb_compose_gather_groups
    ok = gg(B.gpb_gather_group(a, ctypes.pointer(t.c), 1152),
            B.gpb_gather_group(a, ctypes.pointer(t.c), 144))
    assert G(ok, 2, a, a, 0, 64, None, None) == B.OK          # no slots: no launch
    assert G(ok, 0, a, a, 4, 64, None, None) == B.EINVAL
    assert G(ok, 5, a, a, 4, 64, None, None) == B.EINVAL
    assert G(gg(B.gpb_gather_group(a, ctypes.pointer(big.c), 1152)), 1, a, a, 4, 64,
             None, None) == B.EINVAL                           # > 16 table entries
    assert G(gg(B.gpb_gather_group(a, ctypes.pointer(t.c), 1000)), 1, a, a, 4, 64,
             None, None) == B.EALIGN
    assert G(gg(B.gpb_gather_group(a + 8, ctypes.pointer(t.c), 1152)), 1, a, a, 4, 64,
             None, None) == B.EALIGN
    assert G(ok, 2, None, a, 4, 64, None, None) == B.EINVAL
    S = B.lib.gpb_current_row_scatter_groups
    rok = rg(B.gpb_row_group(a, 10, a, 1152), B.gpb_row_group(a, 10, a, 144))
    assert S(rok, 2, a, 0, None, None) == B.OK
    assert S(rok, 2, None, 4, None, None) == B.EINVAL
    assert S(rok, 0, a, 4, None, None) == B.EINVAL
    assert S(rg(B.gpb_row_group(a, 10, a, 100)), 1, a, 4, None, None) == B.EALIGN
    assert S(rg(B.gpb_row_group(a + 4, 10, a, 144)), 1, a, 4, None, None) == B.EALIGN
    assert S(rg(B.gpb_row_group(a, 1 << 40, a, 144)), 1, a, 4, None, None) == B.ERANGE


def test_staging_clear_argument_checks():
    f = B.lib.gpb_staging_clear
    assert f(0x100000, 0, None) == B.OK
    assert f(0x100000, -16, None) == B.EINVAL
    assert f(0x100008, 64, None) == B.EALIGN
    assert f(0x100000, 40, None) == B.EALIGN
    assert f(None, 64, None) == B.EINVAL


_CODE_OF = {oracle.OK: {B.OK}, oracle.BAD_SHAPE: {B.EINVAL, B.EALIGN},
            oracle.BAD_PAGE: {B.EPAGE}, oracle.CAPACITY: {B.ECAPACITY},
            oracle.TOO_LARGE: {B.ERANGE}}


def test_validation_agrees_with_oracle_on_random_batches(orc):
    """Host validation of the library and the oracle accept and reject the
    same batches, for the same reason."""
    rng = np.random.default_rng(7)
    n_bad = 0
    for b in pins_random(rng, 400):
        # break some batches: dummy page, duplicate, range, capacity
        kind = rng.integers(0, 6)
        pages = b.req_pages.copy()
        cap = b.staging_cap_pages
        if kind == 1 and len(pages):
            pages[rng.integers(0, len(pages))] = 0
        elif kind == 2 and len(pages) > 1:
            pages[1] = pages[0]
        elif kind == 3 and len(pages):
            pages[-1] = b.n_pool_pages
        elif kind == 4:
            cap = max(1, cap - b.bs - 1)
        want = orc.validate(b.bs, b.page_size, b.row_bytes, b.n_pool_pages,
                            b.n_pool_entries, b.n_writers, cap, b.prefix_pages,
                            b.cur_tokens, pages)
        m = B.BatchMeta(b.bs, b.page_size, b.row_bytes, b.n_pool_pages, b.n_pool_entries,
                        b.n_writers, cap, b.prefix_pages, b.cur_tokens, pages)
        got = B.lib.gpb_plan_sizes(ctypes.byref(m.c), None, None, None)
        assert got in _CODE_OF[want], (want, got)
        n_bad += want != oracle.OK
    assert n_bad > 50


def pins_random(rng, n):
    return [workloads.random_batch(rng) for _ in range(n)]


def test_package_fails_loudly_without_the_library(tmp_path):
    """With libgpb.so absent the package raises at import: there is no CPU
    path to fall back on."""
    import subprocess
    import sys
    code = ("import os, sys; sys.path.insert(0, %r)\n"
            "try:\n"
            "    import gather_plan_build_amd\n"
            "except ImportError as e:\n"
            "    print('RAISED', e); sys.exit(0)\n"
            "sys.exit(5)\n" % ROOT)
    env = dict(os.environ, GPB_LIB=str(tmp_path / "missing" / "libgpb.so"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "RAISED" in r.stdout and "no fallback" in r.stdout


def test_product_sources_never_reach_the_oracle():
    """The package, its HIP sources and the header name no oracle module,
    file or symbol."""
    import re
    pat = re.compile(r"\boracle\b|gpbo_|liboracle|gpb_oracle")
    roots = [os.path.join(ROOT, "gather_plan_build_amd"), os.path.join(ROOT, "include")]
    hits = []
    for top in roots:
        for dirpath, _, files in os.walk(top):
            for name in files:
                if not name.endswith((".py", ".hip", ".h", ".c", ".cpp")):
                    continue
                path = os.path.join(dirpath, name)
                with open(path, encoding="utf-8") as f:
                    for n, line in enumerate(f, 1):
                        if pat.search(line):
                            hits.append("%s:%d: %s" % (path, n, line.strip()))
    assert not hits, "\n".join(hits)


def test_host_memory_never_reaches_a_kernel():
    """Tensors in host memory and non-GPU devices are refused by the binding
    before any call into the library."""
    import torch
    cpu = torch.zeros(4096, dtype=torch.uint8)
    with pytest.raises(ValueError):
        gpb.staging_clear(cpu)
    with pytest.raises(ValueError):
        B._ptr(cpu)
    b = workloads.make_batch("tiny")
    with pytest.raises(ValueError):
        gpb.Plan(gpb.BatchMeta.of(b), device="cpu")
    pools, curs = workloads.make_values(b, device="cpu")
    with pytest.raises(ValueError):
        gpb.ComposeRunner(gpb.BatchMeta.of(b), pools, curs, device="cpu")


def test_metadata_outside_int32_is_refused():
    with pytest.raises(ValueError):
        gpb.BatchMeta(1, 64, 1152, 16, 1, 1, 4, [2 ** 32 + 1], [0], [1])


def test_plan_key_covers_what_a_plan_depends_on():
    """Two batches share a plan key exactly when their plans are the same:
    the row size may differ, nothing else (layout, spans, table shape,
    staging capacity, page ids)."""
    base = dict(bs=2, page_size=64, row_bytes=1152, n_pool_pages=16, n_pool_entries=1,
                n_writers=1, staging_cap_pages=4, prefix_pages=[1, 1], cur_tokens=[64, 65],
                req_pages=[1, 2, 3, 4, 5])
    key = B.BatchMeta(**base).plan_key()
    assert B.BatchMeta(**dict(base, row_bytes=144)).plan_key() == key
    for change in (dict(page_size=32), dict(n_pool_pages=17), dict(n_pool_entries=2),
                   dict(n_writers=2), dict(staging_cap_pages=5),
                   dict(prefix_pages=[2, 0]), dict(cur_tokens=[65, 64]),
                   dict(req_pages=[1, 2, 3, 5, 4])):
        assert B.BatchMeta(**dict(base, **change)).plan_key() != key, change
