"""CPU oracle for the KV-compose plan build, current-row scatter and slot-dense
page gather.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg are the only users.  Nothing in gather_plan_build_amd/ may
import this package, and this package imports nothing from there.

Two independent routes to the same bytes:

* ``plan`` / ``compose_layer`` run the method's steps in order (C, plain
  loops, gpb_oracle.c): validate, counts, spans, page inverse, staging page
  inverse, gather descriptors, ragged descriptors, staging rows, then per
  layer zero staging, scatter rows, gather pages.
* ``closed_form.dense`` writes the composed dense buffer straight from its
  definition per request (prefix pool rows, current rows, zero tail).

Citations are to the commit pages of the sglang fork (page id = commit hash
in the page address):
  page d63fbd4, commit "current rows written straight into staging" -- the
    staging-direct exchange, index_copy_ fill, [pool || staging] table;
  page d63fbd4, commit "compose_v2" -- -1 descriptors zero-fill;
  page d63fbd4, commit "cut per-layer CPU on the prefill launch path" -- the
    ragged int32 descriptor names and per-batch slot spans;
  page 0d87bc5, commit "prefetch staging exchange" -- page 0 dummy, staging
    slot = batch current index + 1.

Parity status per function (pins in tests/test_oracle_pins.py):
  validate, counts, plan (spans, slot_pages, page_inverse,
  staging_page_inverse, owner, src, writer, staging_rows, mixed_locs),
  compose_layer, closed_form.dense -- pinned (brute force on tagged rows,
  closed form, library special cases, hand-derived worked example);
  token_req -- pinned to numpy repeat (the repeat_interleave the pages used);
  prefix_slots, current_slots, pool_locs, cur_page_token0, cur_page_ntok,
  prefix_desc, current_desc, gather_slots, gather_records, fill -- pinned by
  brute force on tagged rows and against the full gather;
  writer_offsets, writer_tokens, writer_rows, writer_page_row0 -- pinned by
  brute force: one torch index_copy_ per writer into its own slab rebuilds
  the staging the single scatter writes, every token in exactly one list;
  q_lens, kv_lens, q_starts, k_bases, current_bases, q_bases, topk_offsets,
  segments -- the pages give only their names; pinned to the stated
  definitions through the dense and staging geometry they must agree with;
  "parity unpinned" as far as the pages themselves go.
"""
import ctypes

import numpy as np

from . import build as _build
from . import closed_form  # noqa: F401  (re-exported)

_I32P = ctypes.POINTER(ctypes.c_int32)

# validation result codes (gpb_oracle.c)
OK, BAD_SHAPE, BAD_PAGE, CAPACITY, TOO_LARGE = 0, 1, 2, 3, 4

PLAN_FIELDS = ("slot_base", "prefix_span", "current_span", "q_lens", "kv_lens",
               "q_starts", "k_bases", "q_bases", "current_bases", "slot_pages",
               "owner", "src", "page_inverse", "staging_page_inverse", "writer",
               "staging_rows", "mixed_locs", "token_req", "topk_offsets", "segments",
               "prefix_slots", "current_slots", "pool_locs", "cur_page_token0",
               "cur_page_ntok", "prefix_desc", "current_desc", "writer_offsets",
               "writer_tokens", "writer_rows", "writer_page_row0")
# the arrays gpbo_plan writes; the next three come from gpbo_token_expansions,
# the next five from gpbo_prefetch_lists, the two records from
# gpbo_page_records and the last four from gpbo_writer_lists
_PLAN_CORE = PLAN_FIELDS[:-14]


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int64).astype(np.int32))
    return a, a.ctypes.data_as(_I32P)


def _p(a):
    return ctypes.c_void_p(a.ctypes.data if a.size else 0)


class Oracle:
    """The C oracle loaded from one shared library (the default build, or a
    variant built elsewhere, e.g. a planted mistake in a test)."""

    def __init__(self, lib_path):
        lib = ctypes.CDLL(lib_path)
        lib.gpbo_validate.restype = ctypes.c_int
        lib.gpbo_plan.restype = ctypes.c_int
        lib.gpbo_layer.restype = ctypes.c_int
        lib.gpbo_counts.restype = None
        lib.gpbo_token_expansions.restype = None
        lib.gpbo_prefetch_lists.restype = None
        lib.gpbo_gather_slots.restype = ctypes.c_int
        lib.gpbo_fill.restype = ctypes.c_int
        lib.gpbo_page_records.restype = None
        lib.gpbo_gather_records.restype = ctypes.c_int
        lib.gpbo_writer_lists.restype = None
        self.lib = lib
        self.path = lib_path

    def validate(self, bs, page_size, row_bytes, n_pool_pages, n_pool_entries,
                 n_writers, staging_cap_pages, prefix_pages, cur_tokens,
                 req_pages):
        """O1: 0 if the batch is well formed, else a positive reason code."""
        P, pP = _i32(prefix_pages)
        c, pc = _i32(cur_tokens)
        g, pg = _i32(req_pages)
        if bs < 0 or len(P) < bs or len(c) < bs or page_size < 1:
            return BAD_SHAPE
        if (P[:bs] < 0).any() or (c[:bs] < 0).any():
            return BAD_SHAPE
        # gpb_oracle.c reads as many page ids as the batch has pages
        n_pages = int(P[:bs].astype(np.int64).sum()
                      + ((c[:bs].astype(np.int64) + page_size - 1) // page_size).sum())
        if n_pages != len(g):
            return BAD_SHAPE
        return self.lib.gpbo_validate(bs, page_size, row_bytes, n_pool_pages,
                                      n_pool_entries, n_writers,
                                      staging_cap_pages, pP, pc, pg)

    def counts(self, bs, page_size, prefix_pages, cur_tokens):
        """O2: (S, T, NCP) = dense slots, current rows, current pages."""
        P, pP = _i32(prefix_pages)
        c, pc = _i32(cur_tokens)
        out = (ctypes.c_int64 * 3)()
        self.lib.gpbo_counts(bs, page_size, pP, pc, out)
        return int(out[0]), int(out[1]), int(out[2])

    def plan(self, bs, page_size, row_bytes, n_pool_pages, n_pool_entries,
             n_writers, staging_cap_pages, prefix_pages, cur_tokens, req_pages):
        """O3..O9: the per-batch plan as a dict of int32 numpy arrays.

        Raises ValueError(code) when validation fails (fail fast)."""
        rc = self.validate(bs, page_size, row_bytes, n_pool_pages,
                           n_pool_entries, n_writers, staging_cap_pages,
                           prefix_pages, cur_tokens, req_pages)
        if rc != OK:
            raise ValueError(rc)
        S, T, NCP = self.counts(bs, page_size, prefix_pages, cur_tokens)
        sizes = {"slot_base": bs, "prefix_span": 2 * bs, "current_span": 2 * bs,
                 "q_lens": bs, "kv_lens": bs, "q_starts": bs, "k_bases": bs,
                 "q_bases": bs, "current_bases": bs, "slot_pages": S,
                 "owner": S, "src": S, "page_inverse": n_pool_pages,
                 "staging_page_inverse": n_pool_pages, "writer": NCP,
                 "staging_rows": T, "mixed_locs": T, "token_req": T,
                 "topk_offsets": T, "segments": 4 * bs, "prefix_slots": S - NCP,
                 "current_slots": NCP, "pool_locs": T, "cur_page_token0": NCP,
                 "cur_page_ntok": NCP, "prefix_desc": 4 * (S - NCP),
                 "current_desc": 4 * NCP, "writer_offsets": n_writers + 1,
                 "writer_tokens": T, "writer_rows": T, "writer_page_row0": NCP}
        # -7 marks entries the oracle never wrote; each array carries a guard
        # tail as long as itself that must stay untouched
        out = {k: np.full(2 * sizes[k] + 64, -7, dtype=np.int32) for k in PLAN_FIELDS}
        P, pP = _i32(prefix_pages)
        c, pc = _i32(cur_tokens)
        g, pg = _i32(req_pages)
        rc = self.lib.gpbo_plan(bs, page_size, row_bytes, n_pool_pages,
                                n_pool_entries, n_writers, staging_cap_pages,
                                pP, pc, pg,
                                *[out[k].ctypes.data_as(_I32P) for k in _PLAN_CORE])
        if rc != OK:
            raise ValueError(rc)
        self.lib.gpbo_token_expansions(bs, page_size, pP, pc,
                                       out["token_req"].ctypes.data_as(_I32P),
                                       out["topk_offsets"].ctypes.data_as(_I32P),
                                       out["segments"].ctypes.data_as(_I32P))
        self.lib.gpbo_prefetch_lists(bs, page_size, pP, pc, pg,
                                     out["prefix_slots"].ctypes.data_as(_I32P),
                                     out["current_slots"].ctypes.data_as(_I32P),
                                     out["pool_locs"].ctypes.data_as(_I32P),
                                     out["cur_page_token0"].ctypes.data_as(_I32P),
                                     out["cur_page_ntok"].ctypes.data_as(_I32P))
        P_ = lambda k: out[k].ctypes.data_as(_I32P)  # noqa: E731
        self.lib.gpbo_page_records(P_("prefix_slots"), S - NCP, P_("owner"), P_("src"),
                                   P_("prefix_desc"))
        self.lib.gpbo_page_records(P_("current_slots"), NCP, P_("owner"), P_("src"),
                                   P_("current_desc"))
        self.lib.gpbo_writer_lists(bs, page_size, n_writers, staging_cap_pages, pP, pc,
                                   P_("staging_rows"), P_("writer_offsets"),
                                   P_("writer_tokens"), P_("writer_rows"),
                                   P_("writer_page_row0"))
        for k in PLAN_FIELDS:
            assert np.all(out[k][sizes[k]:] == -7), "oracle wrote past " + k
        return {k: out[k][:sizes[k]].copy() for k in PLAN_FIELDS}

    def compose_layer(self, table, cur, staging_rows, owner, src, page_size,
                      row_bytes, staging):
        """O10: one layer.

        ``table``: list of uint8 numpy arrays, one arena per pointer-table
        entry (the staging slabs are views into ``staging``).  ``staging``
        (uint8, whole rows) is zeroed, receives the scattered current rows,
        then the gather reads the table.  Returns (dense uint8
        [n_slots*page_size, row_bytes], bad) where bad flags an out-of-range
        descriptor or staging row."""
        RB = int(row_bytes)
        n_slots = int(len(owner))
        assert staging.dtype == np.uint8 and staging.flags.c_contiguous
        assert staging.size % RB == 0
        cur = np.ascontiguousarray(cur, dtype=np.uint8)
        n_rows = int(len(staging_rows))
        assert cur.size >= n_rows * RB
        dense = np.empty((n_slots * page_size, RB), dtype=np.uint8)
        n_tab = max(len(table), 1)
        ptrs = (ctypes.c_void_p * n_tab)(*[t.ctypes.data for t in table])
        pages = (ctypes.c_int64 * n_tab)(*[t.size // (page_size * RB) for t in table])
        sr, psr = _i32(staging_rows)
        ow, pow_ = _i32(owner)
        sc, psc = _i32(src)
        bad = self.lib.gpbo_layer(ptrs, pages, len(table), _p(staging),
                                  ctypes.c_int64(staging.size // RB), _p(cur),
                                  n_rows, psr, pow_, psc, n_slots, page_size,
                                  RB, _p(dense))
        return dense, bool(bad)


    def gather_slots(self, table, slots, owner, src, page_size, row_bytes, dense):
        """O14: gather the listed slots into ``dense`` (uint8 [S*PS, RB]),
        leaving the others.  Returns the out-of-range flag."""
        RB = int(row_bytes)
        assert dense.dtype == np.uint8 and dense.flags.c_contiguous
        n_tab = max(len(table), 1)
        ptrs = (ctypes.c_void_p * n_tab)(*[t.ctypes.data for t in table])
        pages = (ctypes.c_int64 * n_tab)(*[t.size // (page_size * RB) for t in table])
        sl, psl = _i32(slots)
        ow, pow_ = _i32(owner)
        sc, psc = _i32(src)
        assert len(sl) == 0 or (sl.min() >= 0 and sl.max() < len(ow)
                                and dense.size >= len(ow) * page_size * RB)
        return bool(self.lib.gpbo_gather_slots(ptrs, pages, len(table), psl, len(sl),
                                               pow_, psc, page_size, RB, _p(dense)))

    def gather_records(self, table, records, page_size, row_bytes, dense):
        """O17: gather the pages named by (slot, owner, src, 0) records into
        ``dense`` (uint8 [S*PS, RB]), leaving the other slots.  Returns the
        out-of-range flag."""
        RB = int(row_bytes)
        assert dense.dtype == np.uint8 and dense.flags.c_contiguous
        n_tab = max(len(table), 1)
        ptrs = (ctypes.c_void_p * n_tab)(*[t.ctypes.data for t in table])
        pages = (ctypes.c_int64 * n_tab)(*[t.size // (page_size * RB) for t in table])
        rec, prec = _i32(records)
        assert rec.size % 4 == 0
        n = rec.size // 4
        assert n == 0 or (rec[0::4].min() >= 0
                          and (rec[0::4].max() + 1) * page_size * RB <= dense.size)
        return bool(self.lib.gpbo_gather_records(ptrs, pages, len(table), prec, n,
                                                 page_size, RB, _p(dense)))

    def fill(self, staging, staging_rows, pool, pool_locs, cur, row_bytes):
        """O15: each current row to its staging row and its pool row (uint8
        arrays updated in place).  Returns the out-of-range flag."""
        RB = int(row_bytes)
        for a in (staging, pool):
            assert a.dtype == np.uint8 and a.flags.c_contiguous and a.size % RB == 0
        cur = np.ascontiguousarray(cur, dtype=np.uint8)
        sr, psr = _i32(staging_rows)
        pl_, ppl = _i32(pool_locs)
        assert len(sr) == len(pl_) and cur.size >= len(sr) * RB
        return bool(self.lib.gpbo_fill(_p(staging), ctypes.c_int64(staging.size // RB), psr,
                                       _p(pool), ctypes.c_int64(pool.size // RB), ppl,
                                       _p(cur), len(sr), RB))


def pointer_table(pool, staging, n_pool_entries, n_writers, staging_cap_pages,
                  page_size, row_bytes):
    """The [pool entries || staging slabs] table as a list of arrays: NP
    aliases of the one pool arena (every pool entry is this GPU's pool), then
    W slabs carved one after another from ``staging``, CAP pages each."""
    slab = staging_cap_pages * page_size * row_bytes
    flat = staging.reshape(-1)
    return [pool.reshape(-1)] * n_pool_entries + \
        [flat[w * slab:(w + 1) * slab] for w in range(n_writers)]


_default = None


def default():
    """The oracle built from gpb_oracle.c in this directory."""
    global _default
    if _default is None:
        _default = Oracle(_build.build(force=False))
    return _default


def validate(*a, **k):
    return default().validate(*a, **k)


def counts(*a, **k):
    return default().counts(*a, **k)


def plan(*a, **k):
    return default().plan(*a, **k)


def compose_layer(*a, **k):
    return default().compose_layer(*a, **k)


def plan_for(batch, orc=None):
    """plan() for a workloads.Batch."""
    o = orc or default()
    return o.plan(batch.bs, batch.page_size, batch.row_bytes, batch.n_pool_pages,
                  batch.n_pool_entries, batch.n_writers, batch.staging_cap_pages,
                  batch.prefix_pages, batch.cur_tokens, batch.req_pages)


def layer_for(batch, plan_arrays, pool, cur, staging, orc=None):
    """compose_layer() for a workloads.Batch with its pool arena, current
    rows and staging region (numpy uint8)."""
    o = orc or default()
    table = pointer_table(pool, staging, batch.n_pool_entries, batch.n_writers,
                          batch.staging_cap_pages, batch.page_size,
                          batch.row_bytes)
    return o.compose_layer(table, cur, plan_arrays["staging_rows"],
                           plan_arrays["owner"], plan_arrays["src"],
                           batch.page_size, batch.row_bytes, staging)
