"""The per-batch / per-layer compose loop on one GPU.

Once per batch: build the plan and clear both staging halves (one call, the
clear riding in the plan's first launch).  Per layer l: scatter the layer's
current rows into staging half l mod 2, then gather every dense slot into
dense half l mod 2 through that layer's table of pool entries followed by
staging slabs (page d63fbd4, commit "current rows written straight into
staging": the fill is one index_copy_ into cleared staging and one gather
then fills the whole dense buffer; page d63fbd4, commit
"touched-pages-proportional staging": two parity halves, so a layer never
overwrites buffers the previous layer's consumer may still read).  By
default the two steps share one launch (gpb_compose_layer);
``layer_two_launch`` runs them as two.

On one GPU every pool entry of the table is the layer's own pool arena and
every staging entry is a slab carved from the local staging region; stream
order stands in for the cross-GPU barrier.
"""
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
            # batch's plan: no plan array depends on the row size.  Anything
            # else a plan depends on must match (page 0d87bc5, commit
            # "descriptor cache on the slot-remap objects": no reuse across a
            # different layout, spans, device or capacity).
            B.plan_sizes(meta)
            if plan.key != meta.plan_key():
                raise ValueError("a shared plan must come from the same batch metadata "
                                 "(only the row size may differ)")
            dev = torch.device(device)
            if dev.index is None:
                dev = torch.device("cuda", torch.cuda.current_device())
            if plan.device != dev:
                raise ValueError("a shared plan lives on %s, the runner on %s"
                                 % (plan.device, dev))
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
        self.writer_counts = B.writer_counts(meta)
        self.tables = {}
        for k, pool in enumerate(self.pools):
            for h in range(PARITY):
                base = self.staging[h].data_ptr()
                entries = [(pool, self.n_pool_pages)] * self.np_ + \
                    [(base + w * slab, self.cap) for w in range(self.w)]
                self.tables[(k, h)] = B.Sources(entries)

    def begin_batch(self, stream=None):
        """Plan build (unless the plan belongs to a twin) + clear of both
        staging halves (once per batch), the clear riding in the plan's first
        launch."""
        if self.owns_plan:
            self.plan.build(stream, clear=self.staging_all)
        else:
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
        """One layer: the scatter and the gather in one launch."""
        self.layer_fused(layer, stream)

    def layer_two_launch(self, layer, stream=None):
        """One layer as the scatter launch followed by the gather launch."""
        self.scatter(layer, stream)
        self.gather(layer, stream)

    # Layer-ahead prefetch split (page 0d87bc5, commit "prefetch staging
    # exchange"): the prefix pages of a layer's dense buffer can be gathered
    # ahead of time; the consume step is the scatter (or the fused fill) and
    # the gather of the current pages only.

    def gather_prefix(self, layer, stream=None):
        h, k = layer % PARITY, layer % len(self.pools)
        B.compose_gather_records(self.dense[h], self.tables[(k, h)],
                                 self.plan.t["prefix_desc"], self.S - self.plan.NCP,
                                 self.S, self.ps, self.rb, self.status, stream)

    def gather_current(self, layer, stream=None):
        h, k = layer % PARITY, layer % len(self.pools)
        B.compose_gather_records(self.dense[h], self.tables[(k, h)],
                                 self.plan.t["current_desc"], self.plan.NCP, self.S,
                                 self.ps, self.rb, self.status, stream)

    def layer_fused(self, layer, stream=None):
        """The layer's scatter and gather in one launch."""
        h, k = layer % PARITY, layer % len(self.pools)
        B.compose_layer(self.dense[h], self.tables[(k, h)], self.plan, self.S, self.plan.NCP,
                        self.staging[h], self.staging_rows_total,
                        self.curs[layer % len(self.curs)], self.T, self.ps, self.rb,
                        self.status, stream)

    def layer_fill(self, layer, stream=None):
        """The one-launch layer with the fused fill: the current rows also go
        to their pool rows in the layer's pool arena."""
        h, k = layer % PARITY, layer % len(self.pools)
        pool = self.pools[k]
        B.compose_layer_fill(self.dense[h], self.tables[(k, h)], self.plan, self.S,
                             self.plan.NCP, self.staging[h], self.staging_rows_total, pool,
                             self.n_pool_pages * self.ps, self.curs[layer % len(self.curs)],
                             self.T, self.ps, self.rb, self.status, stream)

    def consume_fused(self, layer, stream=None):
        """The consume half in one launch: the scatter and the gather of the
        current pages."""
        h, k = layer % PARITY, layer % len(self.pools)
        B.compose_consume(self.dense[h], self.tables[(k, h)], self.plan, self.S,
                          self.plan.NCP, self.staging[h], self.staging_rows_total,
                          self.curs[layer % len(self.curs)], self.T, self.ps, self.rb,
                          self.status, stream)

    def ahead(self, layer, stream=None):
        """Layer l's consume and layer l + 1's prefix pages in one launch
        (the table: layer l + 1's pool entries, layer l's staging slabs)."""
        h, hn = layer % PARITY, (layer + 1) % PARITY
        k = (layer + 1) % len(self.pools)
        B.compose_layer_ahead(self.dense[h], self.dense[hn], self.tables[(k, h)], self.plan,
                              self.S, self.plan.NCP, self.staging[h],
                              self.staging_rows_total, self.curs[layer % len(self.curs)],
                              self.T, self.ps, self.rb, self.status, stream)

    def consume_fill(self, layer, stream=None):
        """The consume half in one launch with the fused fill: the current
        rows also go to their pool rows in the layer's pool arena."""
        h, k = layer % PARITY, layer % len(self.pools)
        B.compose_consume_fill(self.dense[h], self.tables[(k, h)], self.plan, self.S,
                               self.plan.NCP, self.staging[h], self.staging_rows_total,
                               self.pools[k], self.n_pool_pages * self.ps,
                               self.curs[layer % len(self.curs)], self.T, self.ps, self.rb,
                               self.status, stream)

    def ahead_fill(self, layer, stream=None):
        """ahead() with the fused fill: layer l's current rows also go to
        their pool rows in layer l's pool arena, while the table names layer
        l + 1's pool entries for the prefix pages."""
        h, hn = layer % PARITY, (layer + 1) % PARITY
        k = (layer + 1) % len(self.pools)
        B.compose_layer_ahead_fill(self.dense[h], self.dense[hn], self.tables[(k, h)],
                                   self.plan, self.S, self.plan.NCP, self.staging[h],
                                   self.staging_rows_total, self.pools[layer % len(self.pools)],
                                   self.n_pool_pages * self.ps,
                                   self.curs[layer % len(self.curs)], self.T, self.ps,
                                   self.rb, self.status, stream)

    def run_layer_ahead(self, n_layers, stream=None, before_prefetch=None,
                        after_consume=None, fill=False):
        """The batch with the layer-ahead prefetch on one stream, one launch
        per layer: the prefix pages of layer 0, then for each layer l its
        consume together with the prefix pages of layer l + 1
        (gpb_compose_layer_ahead), the last layer's consume alone.  The dense
        half layer l + 1 fills was last read by layer l - 1, whose launch
        came before.  With ``fill`` every consume also stores the layer's
        current rows at their pool rows (the _fill launches).  Hooks as in
        run_pipelined, both on ``stream``."""
        self.begin_batch(stream)
        if n_layers == 0:
            return
        if before_prefetch is not None:
            before_prefetch(0, stream)
        self.gather_prefix(0, stream)
        for l in range(n_layers):
            if l + 1 < n_layers:
                if before_prefetch is not None:
                    before_prefetch(l + 1, stream)
                (self.ahead_fill if fill else self.ahead)(l, stream)
            else:
                (self.consume_fill if fill else self.consume_fused)(l, stream)
            if after_consume is not None:
                after_consume(l, stream)

    def writer_rows_of(self, layer):
        """Each writer's own current rows in its list order (what a rank that
        computed them would hold): gathered here from the layer's current
        rows by the plan's writer_tokens.  Input preparation for
        scatter_writers, not part of the compose."""
        cur = self.curs[layer % len(self.curs)].view(-1, self.rb)
        toks = self.plan.t["writer_tokens"].long()
        out, at = [], 0
        for n in self.writer_counts:
            out.append(cur.index_select(0, toks[at:at + int(n)]).contiguous())
            at += int(n)
        return out

    def scatter_writers(self, layer, writer_rows, stream=None):
        """The scatter as W writers would run it, each on its own slab only
        (page d63fbd4, commit "counting barrier + CUDA-IPC gather": one writer
        per current page): writer w copies its rows ``writer_rows[w]`` (in
        its list order) to its list's slab-local staging rows."""
        h = layer % PARITY
        slab_rows = self.cap * self.ps
        slab_bytes = slab_rows * self.rb
        base = self.staging[h]
        rows = self.plan.t["writer_rows"]
        at = 0
        for w, n in enumerate(self.writer_counts):
            n = int(n)
            B.current_row_scatter(base[w * slab_bytes:(w + 1) * slab_bytes], slab_rows,
                                  rows[at:at + n] if n else None, writer_rows[w], n, self.rb,
                                  self.status, stream)
            at += n

    def fill(self, layer, stream=None):
        """Fused current fill: current rows to staging and to their pool rows
        in the layer's pool arena."""
        h, k = layer % PARITY, layer % len(self.curs)
        pool = self.pools[layer % len(self.pools)]
        B.current_row_fill(self.staging[h], self.staging_rows_total,
                           self.plan.t["staging_rows"], pool,
                           self.n_pool_pages * self.ps, self.plan.t["pool_locs"],
                           self.curs[k], self.T, self.rb, self.status, stream)

    def run(self, n_layers, stream=None):
        self.begin_batch(stream)
        for l in range(n_layers):
            self.layer(l, stream)

    def run_pipelined(self, n_layers, stream, side, consume="fused",
                      before_prefetch=None, after_consume=None):
        """The batch with the layer-ahead prefetch (page 0d87bc5, commit
        "prefetch staging exchange"): the prefix pages of layer l + 1 are
        gathered on ``side`` while layer l is consumed on ``stream``; the
        consume of layer l is its current-row fill into staging and the
        gather of its current pages into the dense half whose prefix is
        already there.  Events order the two streams:

        - the prefix gather of layer l waits for the consume of layer l - 2,
          the last user of the same dense half (the parity-half reuse
          distance of page d63fbd4, commit "touched-pages-proportional
          staging");
        - the consume of layer l waits for the prefix gather of layer l.

        ``consume``: "fused" (one launch), "scatter" (scatter, then the
        current-page gather) or "fill" (fused fill into staging and pool,
        then the current-page gather).  ``before_prefetch(l, side)`` runs on
        the side stream just before layer l's prefix gather, and
        ``after_consume(l, stream)`` on the main stream right after layer l's
        consume, before the dense half is handed back (a stand-in for the
        attention that reads it).  Both streams keep the default priority."""
        import torch
        self.begin_batch(stream)
        planned = torch.cuda.Event()
        planned.record(stream)
        side.wait_event(planned)
        free = [None] * PARITY
        ready = [torch.cuda.Event() for _ in range(PARITY)]

        def prefetch(l):
            h = l % PARITY
            if free[h] is not None:
                side.wait_event(free[h])
            if before_prefetch is not None:
                before_prefetch(l, side)
            self.gather_prefix(l, side)
            ready[h].record(side)

        if n_layers > 0:
            prefetch(0)
        for l in range(n_layers):
            if l + 1 < n_layers:
                prefetch(l + 1)
            h = l % PARITY
            stream.wait_event(ready[h])
            if consume == "fused":
                self.consume_fused(l, stream)
            else:
                if consume == "fill":
                    self.fill(l, stream)
                else:
                    self.scatter(l, stream)
                self.gather_current(l, stream)
            if after_consume is not None:
                after_consume(l, stream)
            ev = torch.cuda.Event()
            ev.record(stream)
            free[h] = ev

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


def layer_groups(runners, layer, stream=None):
    """One layer for several row formats sharing one plan (the token KV and
    its index-key twin) in one launch for all of them."""
    r0 = runners[0]
    if any(r.plan is not r0.plan for r in runners[1:]):
        raise ValueError("grouped formats must share one plan")
    h = layer % PARITY
    B.compose_layer_groups(
        [(r.dense[h], r.tables[(layer % len(r.pools), h)], r.staging[h], r.staging_rows_total,
          r.curs[layer % len(r.curs)], r.rb) for r in runners],
        r0.plan, r0.S, r0.plan.NCP, r0.T, r0.ps, r0.status, stream)


def layer_groups_two_launch(runners, layer, stream=None):
    """One layer for several row formats sharing one plan: one scatter launch
    and one gather launch for all of them."""
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
