"""Seeded synthetic batches for the KV-compose path.

Metadata (request lengths, page tables) comes from numpy's
``default_rng(seed)``; row values come from a torch generator seeded with the
same seed, on the device the caller names.  The draw order is fixed: per
request prefix lengths, then current lengths, then the page ids of the whole
batch in one ``choice`` without replacement from [1, n_pool_pages), consumed
request by request (that request's prefix pages, then its current pages).
Page 0 is never drawn: it is the pool's dummy page (page 0d87bc5, commit
"prefetch staging exchange").

The workloads follow the shapes of the traced prefill batches the pages
measure (page d63fbd4, commit "cut per-layer CPU on the prefill launch
path": bs=12 with 44.6K current tokens; 78-layer forward; 64-token pages of
576-wide rows).  That trace is not available, so its shape is drawn here.
"""
from dataclasses import dataclass

import numpy as np
import torch

PAGE = 64          # tokens per KV page
ROW_BF16 = 576     # bf16 values per token row (1152 bytes)


def staging_cap_for(total_cur_tokens, bs, page_size=PAGE):
    """Staging pages per writer slab: the extend-token cap in pages plus one
    page of slack per request plus the reserved slot 0 (page d63fbd4, commit
    "touched-pages-proportional staging": capacity from the admission caps;
    page 0d87bc5: slot 0 reserved)."""
    return -(-int(total_cur_tokens) // page_size) + int(bs) + 1


@dataclass
class Batch:
    name: str
    bs: int
    page_size: int
    row_bytes: int
    n_pool_pages: int
    n_pool_entries: int
    n_writers: int
    staging_cap_pages: int
    prefix_pages: np.ndarray      # int32 [bs], whole pages
    cur_tokens: np.ndarray        # int32 [bs]
    req_pages: np.ndarray         # int32 [sum(P + ceil(c/PS))], request-major
    n_layers: int = 1
    n_rotations: int = 1          # distinct pool/current arenas cycled per layer
    value_kind: str = "bf16_normal"   # or "bytes"
    seed: int = 0

    @property
    def n_req_pages(self):
        return int(len(self.req_pages))

    @property
    def n_cur_tokens(self):
        return int(np.asarray(self.cur_tokens, dtype=np.int64).sum())

    @property
    def staging_rows_total(self):
        return self.n_writers * self.staging_cap_pages * self.page_size


def _pages_needed(P, c, page_size):
    return int(np.sum(P, dtype=np.int64)
               + np.sum((np.asarray(c, dtype=np.int64) + page_size - 1) // page_size))


def _draw_pages(rng, n_pool_pages, n):
    if n == 0:
        return np.zeros(0, dtype=np.int32)
    return rng.choice(np.arange(1, n_pool_pages), size=n, replace=False).astype(np.int32)


def _dirichlet_split(rng, total, k):
    """Split ``total`` tokens over k requests by Dirichlet(1,...,1): floor the
    shares, then give +1 to the largest fractional parts (ties to the lower
    index) until the sum is exact.  Zeros are allowed."""
    share = rng.dirichlet(np.ones(k)) * total
    base = np.floor(share).astype(np.int64)
    rest = int(total - base.sum())
    frac = share - base
    order = sorted(range(k), key=lambda i: (-frac[i], i))
    for i in order[:rest]:
        base[i] += 1
    return base.astype(np.int32)


def make_batch(name, seed=0):
    """The five named workloads."""
    rng = np.random.default_rng(seed)
    if name == "tiny":
        P = np.array([3, 5], np.int32)
        c = np.array([100, 37], np.int32)
        n_pool, np_, w, rb, layers, rot, kind = 256, 1, 1, 2 * ROW_BF16, 1, 1, "bf16_normal"
    elif name in ("medium", "multi_source"):
        P = rng.integers(16, 129, size=4).astype(np.int32)          # 1K-8K tokens
        c = rng.integers(512, 2049, size=4).astype(np.int32)
        n_pool, rb, layers, rot, kind = 16384, 2 * ROW_BF16, 1, 1, "bf16_normal"
        np_ = w = (8 if name == "multi_source" else 1)
    elif name == "traced":
        P = rng.integers(0, 513, size=12).astype(np.int32)          # 0-32K tokens
        c = _dirichlet_split(rng, 44600, 12)
        n_pool, np_, w, rb, layers, rot, kind = 16384, 1, 1, 2 * ROW_BF16, 78, 4, "bf16_normal"
    elif name == "opaque":
        bs = 32
        P = np.zeros(bs, np.int32)
        c = np.zeros(bs, np.int32)
        for r in range(bs):
            # r mod 3: 0 -> zero prefix, 1 -> zero current, 2 -> both present
            if r % 3 != 0:
                P[r] = rng.integers(1, 1025)
            if r % 3 != 1:
                c[r] = rng.integers(1, 2049)
        n_pool, np_, w, rb, layers, rot, kind = 40960, 1, 1, 656, 40, 4, "bytes"
    else:
        raise KeyError(name)
    pages = _draw_pages(rng, n_pool, _pages_needed(P, c, PAGE))
    cap = staging_cap_for(int(c.sum()), len(P))
    return Batch(name, len(P), PAGE, rb, n_pool, np_, w, cap, P, c, pages,
                 n_layers=layers, n_rotations=rot, value_kind=kind, seed=seed)


CONFIGS = ("tiny", "medium", "traced", "multi_source", "opaque")


def random_batch(rng, max_bs=6, max_pool=64, page_size=None, row_bytes=None,
                 n_pool_entries=None, n_writers=None, slack=0):
    """A small random batch for brute-force tests: any mix of zero-prefix,
    zero-current and empty requests, current lengths around page edges."""
    PS = page_size or int(rng.choice([1, 2, 4, 16, 64]))
    RB = row_bytes or int(16 * rng.integers(1, 5))
    bs = int(rng.integers(0, max_bs + 1))
    n_pool = int(rng.integers(2, max_pool + 1))
    edge = [0, 1, PS - 1, PS, PS + 1, 2 * PS - 1, 2 * PS + 1]
    P = np.zeros(bs, np.int32)
    c = np.zeros(bs, np.int32)
    for r in range(bs):
        P[r] = rng.integers(0, 4)
        c[r] = max(0, int(rng.choice(edge)) if rng.random() < 0.6 else int(rng.integers(0, 3 * PS)))
    # shrink until the pages fit in the pool (page 0 excluded)
    while _pages_needed(P, c, PS) > n_pool - 1:
        r = int(rng.integers(0, bs))
        if P[r] > 0:
            P[r] -= 1
        elif c[r] > 0:
            c[r] = max(0, c[r] - PS)
    pages = _draw_pages(rng, n_pool, _pages_needed(P, c, PS))
    NP = n_pool_entries or int(rng.integers(1, 4))
    W = n_writers or int(rng.integers(1, 4))
    cap = staging_cap_for(int(c.sum()), bs, PS) + slack
    return Batch("random", bs, PS, RB, n_pool, NP, W, cap, P, c, pages)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _fill(kind, rows, row_bytes, g, device):
    """One arena of ``rows`` rows, uint8 [rows, row_bytes]."""
    out = torch.empty((rows, row_bytes), dtype=torch.uint8, device=device)
    step = max(1, (1 << 26) // row_bytes)   # bounded temporaries
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        if kind == "bf16_normal":
            v = torch.randn((r1 - r0, row_bytes // 2), generator=g, device=device,
                            dtype=torch.float32).to(torch.bfloat16)
            out[r0:r1] = v.view(torch.uint8)
        else:
            out[r0:r1] = torch.randint(0, 256, (r1 - r0, row_bytes), generator=g,
                                       device=device, dtype=torch.uint8)
    return out


# Rows of the indexer-key twin: a 128-byte fp8 key and a 4-byte fp32 scale per
# token, padded to the 16-byte unit rows move in.  The pages do not give the
# indexer row size; this is a parameter of the twin, not of the method.
INDEX_ROW_BYTES = 144


def make_values(batch, device="cpu", seed=None, rotations=None, row_bytes=None,
                value_kind=None):
    """Pool arenas and current rows, ``rotations`` of each (layer l uses
    index l mod rotations).  Pools: uint8 [n_pool_pages*PS, RB] (bf16 N(0,1)
    bit patterns, or uniform bytes); current rows: uint8 [T, RB].  row_bytes
    and value_kind override the batch's (the index-key twin uses bytes)."""
    rot = batch.n_rotations if rotations is None else rotations
    rb = batch.row_bytes if row_bytes is None else row_bytes
    kind = batch.value_kind if value_kind is None else value_kind
    g = _gen(device, batch.seed if seed is None else seed)
    pools = [_fill(kind, batch.n_pool_pages * batch.page_size, rb, g, device)
             for _ in range(rot)]
    curs = [_fill(kind, batch.n_cur_tokens, rb, g, device) for _ in range(rot)]
    return pools, curs
