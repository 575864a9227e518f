"""GPU tests at the size limits of the C ABI: byte offsets in 64 bits (a pool
above 4 GiB read and filled past the 4 GiB mark, by the gather and by the
one-launch layer), the 2 GiB buffer range of the staging region (rows
written at its very end), and 512 MiB pages.  The
oracle's plain copies on host slices are the reference; only the slices the
test touches are copied back."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

GIB = 1 << 30


def _gpb():
    import gather_plan_build_amd as gpb
    return gpb


def _rand(n, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randint(0, 256, (n,), generator=g, device="cuda", dtype=torch.uint8)


def test_gather_reads_pages_beyond_4_gib(orc):
    gpb = _gpb()
    PS, RB = 64, 1152
    page = PS * RB
    n_pages = (5 * GIB) // page + 1
    pool = _rand(n_pages * page, 1)
    src = np.array([n_pages - 1, 3, n_pages - 2, (4 * GIB) // page + 1, 1], np.int32)
    owner = np.zeros(len(src), np.int32)
    dense = torch.empty(len(src) * page, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpb.compose_gather(dense, [(pool, n_pages)], torch.from_numpy(owner).cuda(),
                       torch.from_numpy(src).cuda(), len(src), PS, RB, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    # reference: the oracle's gather over a table of just the pages read
    host_pages = [pool[int(p) * page:(int(p) + 1) * page].cpu().numpy() for p in src]
    table = [np.concatenate(host_pages)]
    want, bad = orc.compose_layer(table, np.zeros((0, RB), np.uint8), np.zeros(0, np.int32),
                                  owner, np.arange(len(src), dtype=np.int32), PS, RB,
                                  np.zeros(RB, np.uint8))
    assert not bad
    assert np.array_equal(dense.cpu().numpy().reshape(-1, RB), want)


def test_scatter_fills_the_end_of_a_2_gib_staging(orc):
    gpb = _gpb()
    RB = 1152
    n_stag = (2 ** 31 - 1) // RB
    stag = torch.zeros(n_stag * RB, dtype=torch.uint8, device="cuda")
    n_rows = 300
    cur = _rand(n_rows * RB, 2)
    rows = np.concatenate([np.arange(n_stag - 250, n_stag), np.arange(50)]).astype(np.int32)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpb.current_row_scatter(stag, n_stag, torch.from_numpy(rows).cuda(), cur, n_rows, RB,
                            status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    cur_np = cur.cpu().numpy().reshape(n_rows, RB)
    tail = stag[(n_stag - 260) * RB:].cpu().numpy().reshape(-1, RB)
    head = stag[:60 * RB].cpu().numpy().reshape(-1, RB)
    assert not tail[:10].any() and not head[50:].any()
    assert np.array_equal(tail[10:], cur_np[:250])
    assert np.array_equal(head[:50], cur_np[250:])


def test_half_gib_pages(orc):
    gpb = _gpb()
    PS, RB = 8192, 65536
    page = PS * RB
    pool = _rand(3 * page, 3)
    dense = torch.empty(2 * page, dtype=torch.uint8, device="cuda")
    owner = torch.zeros(2, dtype=torch.int32, device="cuda")
    src = torch.tensor([2, 0], dtype=torch.int32, device="cuda")
    gpb.compose_gather(dense, [(pool, 3)], owner, src, 2, PS, RB)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    for slot, p in ((0, 2), (1, 0)):
        for r in np.concatenate([[0, PS - 1], rng.integers(0, PS, 6)]):
            a = dense[slot * page + r * RB:slot * page + (r + 1) * RB].cpu()
            b = pool[p * page + r * RB:p * page + (r + 1) * RB].cpu()
            assert torch.equal(a, b), (slot, r)


def test_fill_writes_pool_rows_beyond_4_gib(orc):
    gpb = _gpb()
    RB = 1152
    n_pool_rows = (5 * GIB) // RB
    pool = torch.zeros(n_pool_rows * RB, dtype=torch.uint8, device="cuda")
    n_rows = 40
    cur = _rand(n_rows * RB, 5)
    stag = torch.zeros(64 * RB, dtype=torch.uint8, device="cuda")
    rows = np.arange(1, n_rows + 1, dtype=np.int32)
    locs = np.concatenate([np.arange(n_pool_rows - 20, n_pool_rows),
                           np.arange(100, 120)]).astype(np.int32)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpb.current_row_fill(stag, 64, torch.from_numpy(rows).cuda(), pool, n_pool_rows,
                         torch.from_numpy(locs).cuda(), cur, n_rows, RB, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    cur_np = cur.cpu().numpy().reshape(n_rows, RB)
    # reference: the oracle's fill into host copies of the touched pool ranges
    lo = pool[(n_pool_rows - 25) * RB:].cpu().numpy().copy()
    mid = pool[95 * RB:125 * RB].cpu().numpy().copy()
    want_lo, want_mid = np.zeros_like(lo), np.zeros_like(mid)
    st = np.zeros(64 * RB, np.uint8)
    sub = np.concatenate([want_mid, want_lo])
    sub_locs = np.concatenate([locs[20:] - 95, locs[:20] - (n_pool_rows - 25) + 30])
    assert not orc.fill(st, rows[np.r_[20:40, 0:20]], sub, sub_locs.astype(np.int32),
                        cur_np[np.r_[20:40, 0:20]], RB)
    assert np.array_equal(mid, sub[:30 * RB]) and np.array_equal(lo, sub[30 * RB:])
    assert np.array_equal(stag.cpu().numpy(), st)


def _limits_runner(prefix_pages, cur_tokens, req_pages, n_pool_pages, PS, RB, seed):
    """A one-rotation runner over a batch with the given page ids; the pool
    is random bytes, the current rows too."""
    import workloads
    gpb = _gpb()
    P = np.array(prefix_pages, np.int32)
    c = np.array(cur_tokens, np.int32)
    b = workloads.Batch("limits", len(P), PS, RB, n_pool_pages, 1, 1,
                        workloads.staging_cap_for(int(c.sum()), len(P), PS), P, c,
                        np.array(req_pages, np.int32))
    pool = _rand(n_pool_pages * PS * RB, seed)
    cur = _rand(int(c.sum()) * RB, seed + 1)
    return gpb.ComposeRunner(gpb.BatchMeta.of(b), [pool], [cur]), pool, cur


def _one_launch_equals_two(r):
    """The one-launch layer against the two-launch layer (each checked
    against the oracle elsewhere) on layers 0 and 1, dense poisoned first."""
    r.begin_batch()
    for layer in (0, 1):
        r.dense[layer % 2].fill_(0xA5)
        r.layer_two_launch(layer)
        want = r.dense[layer % 2].clone()
        r.dense[layer % 2].fill_(0x5A)
        r.layer(layer)
        torch.cuda.synchronize()
        assert torch.equal(r.dense[layer % 2], want), "layer %d differs" % layer
        del want
    assert int(r.status.item()) == 0


def test_one_launch_layer_reads_pages_beyond_4_gib(orc):
    """Prefix pages past the 4 GiB mark of a 5 GiB pool, current pages at
    its start, through the one-launch layer; the prefix rows also against
    the pool's bytes."""
    PS, RB = 64, 1152
    page = PS * RB
    n_pages = (5 * GIB) // page + 1
    hi = n_pages - 1
    # request 0: 3 prefix pages (all past 4 GiB), 2 current pages; request 1:
    # 1 prefix page, 3 current pages
    req = [hi, hi - 7, (4 * GIB) // page + 1, 5, 6, hi - 3, 9, 10, 11]
    r, pool, cur = _limits_runner([3, 1], [100, 130], req, n_pages, PS, RB, 11)
    _one_launch_equals_two(r)
    dense = r.dense_of(1)
    for slot, p in ((0, req[0]), (1, req[1]), (2, req[2]), (5, req[5])):
        for row in (0, 17, PS - 1):
            a = dense[slot * PS + row].cpu()
            b = pool[p * page + row * RB:p * page + (row + 1) * RB].cpu()
            assert torch.equal(a, b), (slot, row)
    # current rows land at dense rows mixed_locs
    ml = r.plan.t["mixed_locs"].cpu().numpy()
    for t in (0, 99, 100, 229):
        assert torch.equal(dense[int(ml[t])].cpu(), cur[t * RB:(t + 1) * RB].cpu())


def test_one_launch_layer_half_gib_pages(orc):
    """512 MiB pages through the one-launch layer: one prefix page, one
    current page of 5,000 rows of 64 KiB, staging halves of 1.5 GiB."""
    PS, RB = 8192, 65536
    r, pool, cur = _limits_runner([1], [5000], [3, 1], 4, PS, RB, 21)
    _one_launch_equals_two(r)
    dense = r.dense_of(0)
    page = PS * RB
    for row in (0, 4095, PS - 1):
        assert torch.equal(dense[row].cpu(), pool[3 * page + row * RB:3 * page + (row + 1) * RB].cpu())
    for j in (0, 2500, 4999):
        assert torch.equal(dense[PS + j].cpu(), cur[j * RB:(j + 1) * RB].cpu())
    for j in (5000, PS - 1):
        assert not dense[PS + j].any()
