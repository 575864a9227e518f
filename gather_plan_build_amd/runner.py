"""The per-batch / per-layer compose loop on one GPU.

Once per batch: build the plan and clear both staging halves.  Per layer l:
scatter the layer's current rows into staging half l mod 2, then gather every
dense slot into dense half l mod 2 through that layer's table of pool entries
followed by staging slabs (page d63fbd4, commit "current rows written
straight into staging": the fill is one index_copy_ into cleared staging and
one gather then fills the whole dense buffer; page d63fbd4, commit
"touched-pages-proportional staging": two parity halves, so a layer never
overwrites buffers the previous layer's consumer may still read).

On one GPU every pool entry of the table is the layer's own pool arena and
every staging entry is a slab carved from the local staging region; stream
order stands in for the cross-GPU barrier.
"""
import numpy as np
import torch

from . import binding as B

PARITY = 2


def _check_arena(t, n_bytes, what):
    """An arena the kernels read whole: contiguous uint8 device memory of
    exactly n_bytes."""
    if not t.is_cuda:
        raise ValueError("%s: the tensor is in host memory, the kernels need device "
                         "memory" % what)
    if t.dtype != torch.uint8 or not t.is_contiguous() or t.numel() != n_bytes:
        raise ValueError("%s: need a contiguous uint8 tensor of %d bytes, got %s %s%s"
                         % (what, n_bytes, t.dtype, tuple(t.shape),
                            "" if t.is_contiguous() else " (not contiguous)"))


class ComposeRunner:
    """Arenas, plan and pointer tables for one batch.

    pools[k], curs[k]: uint8 device tensors [rows, row_bytes]; layer l uses
    index l mod len(pools)."""

    def __init__(self, meta, pools, curs, device="cuda", plan=None):
        b = meta.c
        self.meta = meta
        self.ps, self.rb = b.page_size, b.row_bytes
        self.np_, self.w, self.cap = b.n_pool_entries, b.n_writers, b.staging_cap_pages
        self.n_pool_pages = b.n_pool_pages
        if plan is None:
            plan = B.Plan(meta, device)
        else:
            # a twin row format (e.g. indexer keys next to token KV) reuses the
            # batch's plan: no plan array depends on the row size
            B.plan_sizes(meta)
            m = plan.meta.c
            same = ((m.bs, m.page_size, m.n_pool_pages, m.n_pool_entries, m.n_writers,
                     m.staging_cap_pages) == (b.bs, b.page_size, b.n_pool_pages,
                                              b.n_pool_entries, b.n_writers,
                                              b.staging_cap_pages)
                    and np.array_equal(plan.meta.h_prefix, meta.h_prefix)
                    and np.array_equal(plan.meta.h_cur, meta.h_cur)
                    and np.array_equal(plan.meta.h_req, meta.h_req))
            if not same:
                raise ValueError("a shared plan must come from the same batch metadata "
                                 "(only the row size may differ)")
        self.plan = plan
        self.owns_plan = plan.meta is meta
        self.S, self.T = self.plan.S, self.plan.T
        self.pools, self.curs = list(pools), list(curs)
        if not self.pools or not self.curs:
            raise ValueError("at least one pool arena and one current-row arena")
        for p in self.pools:
            _check_arena(p, self.n_pool_pages * self.ps * self.rb, "pool arena")
        for c in self.curs:
            _check_arena(c, self.T * self.rb, "current rows")
        self.staging_rows_total = self.w * self.cap * self.ps
        slab = self.cap * self.ps * self.rb
        dev = B._gpu_device(device)
        # both parity halves in one allocation, so one launch clears them
        half = self.staging_rows_total * self.rb
        self.staging_all = torch.empty(PARITY * half, dtype=torch.uint8, device=dev)
        self.staging = [self.staging_all[h * half:(h + 1) * half] for h in range(PARITY)]
        self.dense = [torch.empty(max(self.S * self.ps * self.rb, 16), dtype=torch.uint8,
                                  device=dev) for _ in range(PARITY)]
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.tables = {}
        for k, pool in enumerate(self.pools):
            for h in range(PARITY):
                base = self.staging[h].data_ptr()
                entries = [(pool, self.n_pool_pages)] * self.np_ + \
                    [(base + w * slab, self.cap) for w in range(self.w)]
                self.tables[(k, h)] = B.Sources(entries)

    def begin_batch(self, stream=None):
        """Plan build (unless the plan belongs to a twin) + clear of both
        staging halves (once per batch)."""
        if self.owns_plan:
            self.plan.build(stream)
        B.staging_clear(self.staging_all, stream=stream)

    def scatter(self, layer, stream=None):
        h, k = layer % PARITY, layer % len(self.curs)
        B.current_row_scatter(self.staging[h], self.staging_rows_total,
                              self.plan.t["staging_rows"], self.curs[k], self.T,
                              self.rb, self.status, stream)

    def gather(self, layer, stream=None):
        h, k = layer % PARITY, layer % len(self.pools)
        B.compose_gather(self.dense[h], self.tables[(k, h)], self.plan.t["owner"],
                         self.plan.t["src"], self.S, self.ps, self.rb, self.status,
                         stream)

    def layer(self, layer, stream=None):
        self.scatter(layer, stream)
        self.gather(layer, stream)

    # Layer-ahead prefetch split (page 0d87bc5, commit "prefetch staging
    # exchange"): the prefix pages of a layer's dense buffer can be gathered
    # ahead of time; the consume step is the scatter (or the fused fill) and
    # the gather of the current pages only.

    def gather_prefix(self, layer, stream=None):
        h, k = layer % PARITY, layer % len(self.pools)
        t = self.plan.t
        B.compose_gather_slots(self.dense[h], self.tables[(k, h)], t["prefix_slots"],
                               self.S - self.plan.NCP, t["owner"], t["src"], self.S,
                               self.ps, self.rb, self.status, stream)

    def gather_current(self, layer, stream=None):
        h, k = layer % PARITY, layer % len(self.pools)
        t = self.plan.t
        B.compose_gather_slots(self.dense[h], self.tables[(k, h)], t["current_slots"],
                               self.plan.NCP, t["owner"], t["src"], self.S, self.ps,
                               self.rb, self.status, stream)

    def fill(self, layer, stream=None):
        """Fused current fill: current rows to staging and to their pool rows
        in the layer's pool arena."""
        h, k = layer % PARITY, layer % len(self.curs)
        pool = self.pools[layer % len(self.pools)]
        B.current_row_fill(self.staging[h], self.staging_rows_total,
                           self.plan.t["staging_rows"], pool,
                           self.n_pool_pages * self.ps, self.plan.t["pool_locs"],
                           self.curs[k], self.T, self.rb, self.status, stream)

    def layer_split(self, layer, stream=None, fused_fill=False):
        """One layer as prefetch (prefix gather) then consume (fill or
        scatter, then the current-page gather)."""
        self.gather_prefix(layer, stream)
        if fused_fill:
            self.fill(layer, stream)
        else:
            self.scatter(layer, stream)
        self.gather_current(layer, stream)

    def run(self, n_layers, stream=None):
        self.begin_batch(stream)
        for l in range(n_layers):
            self.layer(l, stream)

    def dense_of(self, layer):
        """Dense half written by ``layer`` as [S*PS, RB] uint8 (valid until
        layer + 2 runs)."""
        return self.dense[layer % PARITY][:self.S * self.ps * self.rb].view(-1, self.rb)

    def staging_of(self, layer):
        return self.staging[layer % PARITY].view(-1, self.rb)

    def algorithmic_bytes_per_layer(self):
        """Bytes the compose must move per layer: read and write every dense
        page, read and write every current row, plus the descriptor reads
        (owner/src per slot, staging row per token) and the table."""
        page = self.ps * self.rb
        return (2 * self.S * page + 2 * self.T * self.rb + 8 * self.S + 4 * self.T
                + 8 * (self.np_ + self.w))

    def gather_bytes(self):
        return 2 * self.S * self.ps * self.rb + 8 * self.S

    def scatter_bytes(self):
        return 2 * self.T * self.rb + 4 * self.T


def layer_groups(runners, layer, stream=None):
    """One layer for several row formats sharing one plan (the token KV and
    its index-key twin): one scatter launch and one gather launch for all of
    them."""
    r0 = runners[0]
    if any(r.plan is not r0.plan for r in runners[1:]):
        raise ValueError("grouped formats must share one plan")
    h = layer % PARITY
    t = r0.plan.t
    B.current_row_scatter_groups(
        [(r.staging[h], r.staging_rows_total, r.curs[layer % len(r.curs)], r.rb)
         for r in runners], t["staging_rows"], r0.T, r0.status, stream)
    B.compose_gather_groups(
        [(r.dense[h], r.tables[(layer % len(r.pools), h)], r.rb) for r in runners],
        t["owner"], t["src"], r0.S, r0.ps, r0.status, stream)
