"""Pins for the oracle: checks tied to what the pages and plain mathematics fix,
not to the oracle's own formulas.

* Brute force on tagged rows: every pool row and current row carries its
  origin in its first 8 bytes, so each dense and staging row can be traced
  back to where it came from, and counted.
* Library special cases: the scatter is torch's ``index_copy_`` on uint8
  views (the routine the pages used: page d63fbd4, commit "current rows
  written straight into staging"; page 0d87bc5, commit "fp8 index_copy_ ->
  uint8 views"); the gather is ``index_select`` over the concatenated
  [pool pages || staging pages] arena; a zero-current request is
  ``np.take`` of its prefix pages.
* A worked example derived by hand (the tiny workload).
* Fail-fast validation cases (page 0 dummy, duplicate pages, capacity).

Each ``pin_*`` raises AssertionError on a mismatch.  They take the oracle
instance as an argument so the same checks run against planted mistakes.
"""
import numpy as np
import torch

import oracle
from oracle import closed_form

KIND_POOL, KIND_CUR = 1, 2
_MASK = (1 << 40) - 1


def _tag_rows(arr, kind):
    idx = np.arange(arr.shape[0], dtype=np.int64)
    tags = (np.int64(kind) << 40) | idx
    arr[:, :8] = tags.astype("<i8").view(np.uint8).reshape(-1, 8)


def tagged_values(batch, seed=1234):
    """uint8 pool [n_pool_pages*PS, RB] and current rows [T, RB]; bytes 0..7
    of each row hold (kind << 40 | row index), the rest are random."""
    rng = np.random.default_rng(seed)
    PS, RB = batch.page_size, batch.row_bytes
    pool = rng.integers(0, 256, (batch.n_pool_pages * PS, RB), dtype=np.uint8)
    cur = rng.integers(0, 256, (batch.n_cur_tokens, RB), dtype=np.uint8)
    _tag_rows(pool, KIND_POOL)
    _tag_rows(cur, KIND_CUR)
    return pool, cur


def decode(rows):
    """(kind, index) per row; kind 0 means an all-zero row."""
    if rows.shape[0] == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    v = np.ascontiguousarray(rows[:, :8]).view("<i8").reshape(-1)
    kind = v >> 40
    idx = v & _MASK
    zero = ~rows.any(axis=1)
    kind = np.where(zero, 0, kind)
    assert np.all((kind == 0) | (kind == KIND_POOL) | (kind == KIND_CUR)), \
        "a dense row matches no source row"
    return kind, np.where(zero, -1, idx)


def run_layer(orc, batch, pool, cur, dirty=0xAB):
    """Plan + one layer through the oracle; staging starts dirty so a missing
    zero fill shows."""
    pl = oracle.plan_for(batch, orc)
    staging = np.full(batch.staging_rows_total * batch.row_bytes, dirty, np.uint8)
    dense, bad = oracle.layer_for(batch, pl, pool, cur, staging, orc)
    assert not bad, "a valid plan produced an out-of-range descriptor"
    return pl, dense, staging.reshape(-1, batch.row_bytes)


def pin_dense_brute_force(batch, dense):
    """Walk every request and every dense row: prefix rows are the listed pool
    pages row by row, then the request's current tokens in order, then zero
    rows up to the page boundary; every source row appears exactly once."""
    PS = batch.page_size
    kind, idx = decode(dense)
    row = 0
    cursor = 0
    token = 0
    for P, c in zip(batch.prefix_pages.tolist(), batch.cur_tokens.tolist()):
        pages = -(-c // PS)
        for k in range(P):
            page = int(batch.req_pages[cursor + k])
            for j in range(PS):
                assert kind[row] == KIND_POOL and idx[row] == page * PS + j, \
                    "prefix row %d holds the wrong pool row" % row
                row += 1
        for j in range(pages * PS):
            if j < c:
                assert kind[row] == KIND_CUR and idx[row] == token + j, \
                    "current row %d holds the wrong token" % row
            else:
                assert kind[row] == 0, "tail row %d of a current page is not zero" % row
            row += 1
        cursor += P + pages
        token += c
    assert row == dense.shape[0], "dense buffer has rows beyond the batch"
    # every source row written exactly once
    used = idx[kind == KIND_POOL]
    assert len(np.unique(used)) == len(used)
    toks = idx[kind == KIND_CUR]
    assert np.array_equal(np.sort(toks), np.arange(batch.n_cur_tokens))


def pin_closed_form(batch, pool, cur, dense):
    ref = closed_form.dense(pool, cur, batch.prefix_pages, batch.cur_tokens,
                            batch.req_pages, batch.page_size)
    assert np.array_equal(ref, dense), "oracle dense differs from the closed form"


def pin_plan_geometry(batch, pl, dense, staging):
    """Every plan array against the dense and staging rows it describes."""
    PS, RB = batch.page_size, batch.row_bytes
    NP, W, CAP = batch.n_pool_entries, batch.n_writers, batch.staging_cap_pages
    bs = batch.bs
    P = batch.prefix_pages.astype(np.int64)
    c = batch.cur_tokens.astype(np.int64)
    S = dense.shape[0] // PS
    T = batch.n_cur_tokens
    kind, idx = decode(dense)
    skind, sidx = decode(staging)
    ps_ = pl["prefix_span"].reshape(-1, 2) if bs else np.zeros((0, 2), np.int32)
    cs_ = pl["current_span"].reshape(-1, 2) if bs else np.zeros((0, 2), np.int32)

    # spans abut and tile [0, S) in request order
    at = 0
    for r in range(bs):
        assert ps_[r, 0] == at and ps_[r, 1] - ps_[r, 0] == P[r]
        assert cs_[r, 0] == ps_[r, 1]
        at = cs_[r, 1]
        assert pl["slot_base"][r] == ps_[r, 0]
    assert at == S

    # slot_pages / page_inverse (a true inverse, S entries set)
    sp = pl["slot_pages"]
    for r in range(bs):
        for s in range(ps_[r, 0], ps_[r, 1]):
            rows = slice(s * PS, (s + 1) * PS)
            assert np.all(kind[rows] == KIND_POOL) and np.all(idx[rows] // PS == sp[s])
    assert np.array_equal(np.sort(sp), np.sort(batch.req_pages))
    inv = pl["page_inverse"]
    assert (inv != -1).sum() == S
    for s in range(S):
        assert inv[sp[s]] == s

    # token geometry: q_starts/q_lens tile [0, T); mixed_locs is the dense row
    at = 0
    for r in range(bs):
        assert pl["q_starts"][r] == at and pl["q_lens"][r] == c[r]
        at += c[r]
    assert at == T
    ml = pl["mixed_locs"]
    assert np.all(kind[ml] == KIND_CUR) and np.array_equal(idx[ml], np.arange(T))

    # per-token expansions: request row ids are numpy's repeat of the request
    # index over the token counts; the top-k offset of a token is the first
    # dense row of its request, so offset + KV position lands on the row that
    # holds that position (prefix row x, or the token itself)
    assert np.array_equal(pl["token_req"], np.repeat(np.arange(bs), c).astype(np.int32))
    seg = pl["segments"].reshape(-1, 4) if bs else np.zeros((0, 4), np.int32)
    sp_all = pl["slot_pages"]
    for r in range(bs):
        toks = np.nonzero(pl["token_req"] == r)[0]
        base = pl["topk_offsets"][toks]
        assert np.all(base == seg[r, 2])
        assert seg[r, 0] == (toks[0] if len(toks) else seg[r, 0]) and seg[r, 1] == c[r]
        assert seg[r, 3] == pl["kv_lens"][r] and seg[r, 2] == pl["k_bases"][r]
        for jj, t in enumerate(toks):
            row = base[jj] + PS * P[r] + jj
            assert kind[row] == KIND_CUR and idx[row] == t
        for x in range(0, PS * P[r], max(1, PS // 2)):
            row = seg[r, 2] + x
            assert kind[row] == KIND_POOL
            assert idx[row] == sp_all[ps_[r, 0] + x // PS] * PS + x % PS
    at = 0
    for r in range(bs):
        assert seg[r, 0] == at
        at += c[r]

    # dense bases: each request owns rows [k_bases, k_bases + PS*n_r); its
    # current rows start at current_bases; kv_lens counts its non-pad rows
    for r in range(bs):
        kb = pl["k_bases"][r]
        assert kb == PS * ps_[r, 0]
        end = PS * cs_[r, 1]
        region = slice(kb, end)
        assert pl["kv_lens"][r] == int((kind[region] != 0).sum())
        assert pl["current_bases"][r] == PS * cs_[r, 0]
        if c[r] > 0:
            assert kind[pl["current_bases"][r]] == KIND_CUR
            assert idx[pl["current_bases"][r]] == pl["q_starts"][r]

    # current pages in batch order: writer round-robin, slot = index + 1
    owner, src = pl["owner"], pl["src"]
    i = 0
    for r in range(bs):
        if c[r] > 0:
            # q_bases: page-padded current base = PS * (batch index of the
            # request's first current page)
            assert pl["q_bases"][r] == PS * (src[cs_[r, 0]] - 1)
        for s in range(cs_[r, 0], cs_[r, 1]):
            assert pl["writer"][i] == i % W, "writers are not round-robin"
            assert owner[s] == NP + pl["writer"][i] and src[s] == i + 1
            i += 1
        for s in range(ps_[r, 0], ps_[r, 1]):
            assert 0 <= owner[s] < NP and owner[s] == sp[s] % NP and src[s] == sp[s]
        if c[r] == 0:
            assert np.all(owner[ps_[r, 0]:cs_[r, 1]] < NP)
        if P[r] == 0:
            assert np.all(owner[ps_[r, 0]:cs_[r, 1]] >= NP)
    assert i == len(pl["writer"])
    at = 0
    for r in range(bs):
        if c[r] == 0:
            assert pl["q_bases"][r] == at
        at += PS * (cs_[r, 1] - cs_[r, 0])
    if W == 1:
        for r in range(bs):
            if c[r] > 0:
                assert pl["staging_rows"][pl["q_starts"][r]] == PS + pl["q_bases"][r]

    # staging rows: injective, inside the carved slabs, never slot 0 of a
    # slab, and the staging holds exactly the current rows there, zeros else
    sr = pl["staging_rows"].astype(np.int64)
    assert np.all(sr >= 0) and np.all(sr < W * CAP * PS)
    assert len(np.unique(sr)) == T
    assert np.all(sr % (CAP * PS) >= PS), "a current row landed in slot 0"
    assert np.all(skind[sr] == KIND_CUR) and np.array_equal(sidx[sr], np.arange(T))
    others = np.ones(staging.shape[0], bool)
    others[sr] = False
    assert np.all(skind[others] == 0), "staging rows outside the scatter are not zero"

    # staging_page_inverse: current page -> carved staging page of its rows
    spi = pl["staging_page_inverse"]
    cur_pages = set()
    for r in range(bs):
        for s in range(cs_[r, 0], cs_[r, 1]):
            cur_pages.add(int(sp[s]))
    for p in range(batch.n_pool_pages):
        if p not in cur_pages:
            assert spi[p] == -1
    t = 0
    for r in range(bs):
        for j in range(c[r]):
            page = sp[cs_[r, 0] + j // PS]
            assert spi[page] == sr[t] // PS
            t += 1
    assert RB % 16 == 0


def pin_library_routines(batch, pl, pool, cur, dense, staging):
    """Scatter == torch index_copy_ on uint8 rows; gather == index_select over
    the concatenated [pool pages || staging pages]; zero-current requests ==
    np.take of their prefix pages."""
    PS, RB = batch.page_size, batch.row_bytes
    NP, CAP = batch.n_pool_entries, batch.staging_cap_pages
    ref = torch.zeros((batch.staging_rows_total, RB), dtype=torch.uint8)
    ref.index_copy_(0, torch.from_numpy(pl["staging_rows"].astype(np.int64)),
                    torch.from_numpy(np.ascontiguousarray(cur)))
    assert np.array_equal(ref.numpy(), staging), "scatter != index_copy_"

    pool_pages = torch.from_numpy(pool.reshape(batch.n_pool_pages, PS * RB))
    stag_pages = torch.from_numpy(np.ascontiguousarray(staging).reshape(-1, PS * RB))
    arena = torch.cat([pool_pages, stag_pages], 0)
    owner = pl["owner"].astype(np.int64)
    src = pl["src"].astype(np.int64)
    flat = np.where(owner < NP, src, batch.n_pool_pages + (owner - NP) * CAP + src)
    got = torch.index_select(arena, 0, torch.from_numpy(flat))
    assert np.array_equal(got.numpy().reshape(-1, RB), dense), "gather != index_select"

    ps_ = pl["prefix_span"].reshape(-1, 2)
    for r in range(batch.bs):
        if batch.cur_tokens[r] == 0 and batch.prefix_pages[r] > 0:
            a, b = ps_[r]
            want = np.take(pool.reshape(batch.n_pool_pages, PS * RB),
                           pl["slot_pages"][a:b], axis=0).reshape(-1, RB)
            assert np.array_equal(dense[a * PS:b * PS], want)


def pin_prefetch_split(orc, batch, pl, pool, cur, dense, staging):
    """The layer-ahead split (page 0d87bc5, commit "prefetch staging
    exchange"): the prefix slots and the current slots partition the dense
    slots; gathering the prefix slots first and the current slots second
    reproduces the one-shot gather and leaves the other half untouched; the
    fused fill writes every current row to its staging row and to its pool
    location, and the pool location is the pool row the dense buffer shows
    for that token's page."""
    PS, RB = batch.page_size, batch.row_bytes
    NP = batch.n_pool_entries
    S = dense.shape[0] // PS
    kind, idx = decode(dense)
    pre, cur_s = pl["prefix_slots"], pl["current_slots"]
    assert len(pre) + len(cur_s) == S
    assert np.array_equal(np.sort(np.concatenate([pre, cur_s])), np.arange(S))
    assert np.all(np.diff(pre) > 0) and np.all(np.diff(cur_s) > 0)
    for s in pre:
        assert np.all(kind[s * PS:(s + 1) * PS] == KIND_POOL)
    for i, s in enumerate(cur_s):
        assert np.all(kind[s * PS:(s + 1) * PS] != KIND_POOL)
        assert pl["owner"][s] >= NP and pl["src"][s] == i + 1
    ml = pl["mixed_locs"].astype(np.int64)
    # the tokens a current page holds: exactly those whose dense row is in it
    for i, s in enumerate(cur_s):
        toks = np.nonzero(ml // PS == s)[0]
        assert pl["cur_page_ntok"][i] == len(toks) and 1 <= len(toks) <= PS
        assert pl["cur_page_token0"][i] == toks[0] and np.all(np.diff(toks) == 1)
    locs = pl["pool_locs"].astype(np.int64)
    assert np.array_equal(locs // PS, pl["slot_pages"][ml // PS])
    assert np.array_equal(locs % PS, ml % PS)

    table = oracle.pointer_table(pool, staging.reshape(-1), NP, batch.n_writers,
                                 batch.staging_cap_pages, PS, RB)
    split = np.full_like(dense, 0xEE)
    assert not orc.gather_slots(table, pre, pl["owner"], pl["src"], PS, RB, split)
    for s in cur_s:
        assert np.all(split[s * PS:(s + 1) * PS] == 0xEE), "prefix gather touched a current slot"
    assert not orc.gather_slots(table, cur_s, pl["owner"], pl["src"], PS, RB, split)
    assert np.array_equal(split, dense), "split gather != one-shot gather"

    st = np.zeros(batch.staging_rows_total * RB, np.uint8)
    pool2 = pool.copy()
    assert not orc.fill(st, pl["staging_rows"], pool2.reshape(-1), pl["pool_locs"], cur, RB)
    assert np.array_equal(st.reshape(-1, RB), staging), "fill staging != scatter staging"
    touched = np.zeros(pool.shape[0], bool)
    touched[locs] = True
    assert np.array_equal(pool2[~touched], pool[~touched])
    pk, pi = decode(pool2[locs])
    assert np.all(pk == KIND_CUR) and np.array_equal(pi, np.arange(len(locs)))


def pin_page_records(orc, batch, pl, pool, dense, staging):
    """The gather records of the two split halves: their slots are the prefix
    and current slot lists, each record names the page the one-shot gather
    puts in that slot, and gathering the prefix records then the current
    records (O17) rebuilds the one-shot dense buffer, the first pass leaving
    every current slot untouched."""
    PS, RB = batch.page_size, batch.row_bytes
    pre = pl["prefix_desc"].reshape(-1, 4)
    cur = pl["current_desc"].reshape(-1, 4)
    assert np.array_equal(pre[:, 0], pl["prefix_slots"])
    assert np.array_equal(cur[:, 0], pl["current_slots"])
    assert not pre[:, 3].any() and not cur[:, 3].any()
    kind, idx = decode(dense)
    table = oracle.pointer_table(pool, staging.reshape(-1), batch.n_pool_entries,
                                 batch.n_writers, batch.staging_cap_pages, PS, RB)
    # each record's (owner, src) addresses exactly the rows its slot holds
    for s, e, p, _ in np.concatenate([pre, cur]):
        arena = table[e].reshape(-1, RB)
        assert np.array_equal(arena[p * PS:(p + 1) * PS], dense[s * PS:(s + 1) * PS])
    split = np.full_like(dense, 0xEE)
    assert not orc.gather_records(table, pre.reshape(-1), PS, RB, split)
    for s in cur[:, 0]:
        assert np.all(split[s * PS:(s + 1) * PS] == 0xEE), "prefix records touched a current slot"
    assert not orc.gather_records(table, cur.reshape(-1), PS, RB, split)
    assert np.array_equal(split, dense), "record gather != one-shot gather"


def pin_writer_lists(batch, pl, cur, staging):
    """Per-writer scatter lists (page d63fbd4, commit "counting barrier +
    CUDA-IPC gather": one writer per current page; page 0d87bc5, commit
    "prefetch staging exchange": each rank fills its own rows into its own
    staging).  Every token sits in exactly one list, in token order, in the
    list of its page's writer; one torch index_copy_ per writer of its own
    rows into its own slab rebuilds exactly the staging the single scatter
    wrote; a page's first entry holds the page's first token."""
    PS, RB = batch.page_size, batch.row_bytes
    W, CAP = batch.n_writers, batch.staging_cap_pages
    T = batch.n_cur_tokens
    off = pl["writer_offsets"].astype(np.int64)
    toks = pl["writer_tokens"].astype(np.int64)
    rows = pl["writer_rows"].astype(np.int64)
    assert len(off) == W + 1 and off[0] == 0 and off[-1] == T
    assert np.all(np.diff(off) >= 0)
    assert np.array_equal(np.sort(toks), np.arange(T)), "a token is missing or repeated"
    slab_rows = CAP * PS
    cur_t = torch.from_numpy(np.ascontiguousarray(cur))
    rebuilt = []
    for w in range(W):
        seg = slice(off[w], off[w + 1])
        tw, rw = toks[seg], rows[seg]
        assert np.all(np.diff(tw) > 0), "list %d is not in token order" % w
        assert np.all((rw >= PS) & (rw < slab_rows)), "a row outside slab %d" % w
        assert np.array_equal(rw + w * slab_rows, pl["staging_rows"][tw])
        slab = torch.zeros((slab_rows, RB), dtype=torch.uint8)
        slab.index_copy_(0, torch.from_numpy(rw), cur_t[torch.from_numpy(tw)])
        rebuilt.append(slab.numpy())
    if W:
        assert np.array_equal(np.concatenate(rebuilt), staging), \
            "per-writer scatters != the single scatter"
    # page i's tokens are entries writer_page_row0[i] ... of its writer's list
    for i, (t0, n) in enumerate(zip(pl["cur_page_token0"], pl["cur_page_ntok"])):
        w = pl["writer"][i]
        k = off[w] + pl["writer_page_row0"][i]
        assert np.array_equal(toks[k:k + n], np.arange(t0, t0 + n))


def check_batch(orc, batch):
    """All per-batch pins on one batch."""
    pool, cur = tagged_values(batch)
    pl, dense, staging = run_layer(orc, batch, pool, cur)
    pin_dense_brute_force(batch, dense)
    pin_closed_form(batch, pool, cur, dense)
    pin_plan_geometry(batch, pl, dense, staging)
    pin_library_routines(batch, pl, pool, cur, dense, staging)
    pin_prefetch_split(orc, batch, pl, pool, cur, dense, staging)
    pin_page_records(orc, batch, pl, pool, dense, staging)
    pin_writer_lists(batch, pl, cur, staging)


def pin_tiny_worked(orc):
    """The tiny workload by hand: P = (3, 5) pages, c = (100, 37) tokens,
    64-token pages.  C = (2, 1) current pages, n = (5, 6) slots, S = 11,
    T = 137, three current pages (batch indices 0, 1 for request 0 and 2 for
    request 1, staging slots 1, 2, 3)."""
    import workloads
    b = workloads.make_batch("tiny")
    pl = oracle.plan_for(b, orc)
    g = b.req_pages
    assert orc.counts(b.bs, 64, b.prefix_pages, b.cur_tokens) == (11, 137, 3)
    assert pl["slot_base"].tolist() == [0, 5]
    assert pl["prefix_span"].tolist() == [0, 3, 5, 10]
    assert pl["current_span"].tolist() == [3, 5, 10, 11]
    assert pl["q_lens"].tolist() == [100, 37]
    assert pl["kv_lens"].tolist() == [3 * 64 + 100, 5 * 64 + 37]       # 292, 357
    assert pl["q_starts"].tolist() == [0, 100]
    assert pl["k_bases"].tolist() == [0, 5 * 64]                        # 0, 320
    assert pl["current_bases"].tolist() == [3 * 64, 5 * 64 + 5 * 64]    # 192, 640
    assert pl["q_bases"].tolist() == [0, 2 * 64]                        # 0, 128
    assert pl["slot_pages"].tolist() == g.tolist()
    assert pl["owner"].tolist() == [0, 0, 0, 1, 1, 0, 0, 0, 0, 0, 1]
    assert pl["src"].tolist() == g[:3].tolist() + [1, 2] + g[5:10].tolist() + [3]
    assert pl["writer"].tolist() == [0, 0, 0]
    want_rows = [64 + t for t in range(100)] + [192 + j for j in range(37)]
    assert pl["staging_rows"].tolist() == want_rows
    assert pl["mixed_locs"].tolist() == [192 + t for t in range(100)] + \
        [640 + j for j in range(37)]
    inv = pl["page_inverse"]
    assert [int(inv[p]) for p in g] == list(range(11))
    assert (inv == -1).sum() == 256 - 11
    spi = pl["staging_page_inverse"]
    assert (int(spi[g[3]]), int(spi[g[4]]), int(spi[g[10]])) == (1, 2, 3)
    assert (spi == -1).sum() == 256 - 3
    # dense rows [292, 320) and [677, 704) are the zero tails
    pool, cur = tagged_values(b)
    _, dense, _ = run_layer(orc, b, pool, cur)
    zero = ~dense.any(axis=1)
    assert zero.sum() == (320 - 292) + (704 - 677)
    assert zero[292:320].all() and zero[677:704].all()


def pin_validation(orc):
    """Fail-fast rejections (page 0 is the dummy page; pages are distinct;
    staging holds slot 0 plus every current page; rows are 16-byte units)."""
    v = orc.validate
    ok = dict(bs=2, page_size=64, row_bytes=1152, n_pool_pages=16,
              n_pool_entries=1, n_writers=1, staging_cap_pages=4)
    P, c = [1, 1], [64, 65]        # 1 + 2 pages current... 1 + 1 + 2 = 4 pages
    assert v(**ok, prefix_pages=P, cur_tokens=c, req_pages=[1, 2, 3, 4, 5]) == oracle.OK
    assert v(**ok, prefix_pages=P, cur_tokens=c, req_pages=[0, 2, 3, 4, 5]) == oracle.BAD_PAGE
    assert v(**ok, prefix_pages=P, cur_tokens=c, req_pages=[1, 2, 3, 4, 1]) == oracle.BAD_PAGE
    assert v(**ok, prefix_pages=P, cur_tokens=c, req_pages=[1, 2, 3, 4, 16]) == oracle.BAD_PAGE
    assert v(**ok, prefix_pages=P, cur_tokens=c, req_pages=[1, 2, 3, 4, 15]) == oracle.OK
    # three current pages need four staging pages (slot 0 reserved)
    tight = dict(ok, staging_cap_pages=3)
    assert v(**tight, prefix_pages=P, cur_tokens=c, req_pages=[1, 2, 3, 4, 5]) == oracle.CAPACITY
    assert v(**dict(ok, row_bytes=1000), prefix_pages=P, cur_tokens=c,
             req_pages=[1, 2, 3, 4, 5]) == oracle.BAD_SHAPE
    assert v(**ok, prefix_pages=[1, -1], cur_tokens=c, req_pages=[1, 2, 3]) == oracle.BAD_SHAPE
    assert v(**dict(ok, bs=0), prefix_pages=[], cur_tokens=[], req_pages=[]) == oracle.OK
    assert v(**dict(ok, n_writers=0), prefix_pages=P, cur_tokens=c,
             req_pages=[1, 2, 3, 4, 5]) == oracle.BAD_SHAPE


def pin_sentinels(orc):
    """-1 descriptors zero-fill their page (page d63fbd4, commit "compose_v2");
    out-of-range descriptors and staging rows are flagged, never read."""
    PS, RB = 4, 32
    rng = np.random.default_rng(5)
    pool = rng.integers(1, 256, (8 * PS, RB), dtype=np.uint8)
    staging = np.full(3 * PS * RB, 0x5A, np.uint8)
    cur = rng.integers(1, 256, (2, RB), dtype=np.uint8)
    table = [pool.reshape(-1), staging]
    owner = np.array([-1, 0, 0, -1, 0], np.int32)
    src = np.array([3, -1, 2, -1, 7], np.int32)
    dense, bad = orc.compose_layer(table, cur, np.array([5, 9], np.int32), owner, src,
                                   PS, RB, staging)
    assert not bad
    d = dense.reshape(5, PS, RB)
    assert not d[0].any() and not d[1].any() and not d[3].any()
    assert np.array_equal(d[2].reshape(-1, RB), pool[2 * PS:3 * PS])
    assert np.array_equal(d[4].reshape(-1, RB), pool[7 * PS:8 * PS])
    st = staging.reshape(-1, RB)
    assert np.array_equal(st[5], cur[0]) and np.array_equal(st[9], cur[1])
    assert (st.any(axis=1)).sum() == 2
    # out of range: owner past the table, src past the arena, stray row
    dense, bad = orc.compose_layer(table, cur, np.array([5, 9], np.int32),
                                   np.array([2], np.int32), np.array([0], np.int32),
                                   PS, RB, staging)
    assert bad and not dense.any()
    dense, bad = orc.compose_layer(table, cur, np.array([5, 9], np.int32),
                                   np.array([0], np.int32), np.array([8], np.int32),
                                   PS, RB, staging)
    assert bad and not dense.any()
    dense, bad = orc.compose_layer(table, cur, np.array([-1, 3 * PS], np.int32),
                                   np.array([1], np.int32), np.array([0], np.int32),
                                   PS, RB, staging)
    assert bad and not staging.any()


def random_batches(n, seed=0, **kw):
    import workloads
    rng = np.random.default_rng(seed)
    return [workloads.random_batch(rng, **kw) for _ in range(n)]


def run_all(orc, n_random=60, seed=0):
    """Every pin; used by the pin tests and by the planted-mistake tests."""
    pin_tiny_worked(orc)
    pin_validation(orc)
    pin_sentinels(orc)
    for b in random_batches(n_random, seed=seed):
        check_batch(orc, b)
    for b in random_batches(max(4, n_random // 6), seed=seed + 1, n_writers=3,
                            n_pool_entries=2, page_size=4):
        check_batch(orc, b)
