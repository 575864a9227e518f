"""ctypes binding of libgpb.so (the C ABI in include/gpb.h).

Argument marshalling only: every step of the compose path runs in the HIP
kernels behind the C calls.  torch provides device memory and streams.  The
functions keep the C names without the ``gpb_`` prefix.

There is no fallback: if libgpb.so is missing or fails to load, importing this
module raises.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GPB_LIB", os.path.join(HERE, "libgpb.so"))

MAX_SOURCES = 64
STATUS_BAD_DESCRIPTOR = 1
STATUS_BAD_STAGING_ROW = 2
STATUS_BAD_PLAN_INPUT = 4
STATUS_LAYER_MISMATCH = 8

OK, EINVAL, EALIGN, EPAGE, ECAPACITY, ERANGE, EHIP, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
SCRATCH_BYTES = 64 * 1024 * 1024  # GPB_SCRATCH_BYTES

_I32P = ctypes.POINTER(ctypes.c_int32)


class gpb_batch(ctypes.Structure):
    _fields_ = [("bs", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("row_bytes", ctypes.c_int32), ("n_pool_pages", ctypes.c_int32),
                ("n_pool_entries", ctypes.c_int32), ("n_writers", ctypes.c_int32),
                ("staging_cap_pages", ctypes.c_int32),
                ("h_prefix_pages", ctypes.c_void_p), ("h_cur_tokens", ctypes.c_void_p),
                ("h_req_pages", ctypes.c_void_p), ("d_prefix_pages", ctypes.c_void_p),
                ("d_cur_tokens", ctypes.c_void_p), ("d_req_pages", ctypes.c_void_p)]


PLAN_FIELDS = ("slot_base", "prefix_span", "current_span", "q_lens", "kv_lens",
               "q_starts", "k_bases", "q_bases", "current_bases", "slot_pages",
               "owner", "src", "page_inverse", "staging_page_inverse", "writer",
               "staging_rows", "mixed_locs", "token_req", "topk_offsets", "segments",
               "prefix_slots", "current_slots", "pool_locs", "cur_page_token0",
               "cur_page_ntok", "prefix_desc", "current_desc", "writer_offsets",
               "writer_tokens", "writer_rows", "writer_page_row0")


class gpb_plan(ctypes.Structure):
    _fields_ = [("d_" + f, ctypes.c_void_p) for f in PLAN_FIELDS] + \
        [("d_status", ctypes.c_void_p)]


class gpb_sources(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32),
                ("base", ctypes.c_void_p * MAX_SOURCES),
                ("n_pages", ctypes.c_int64 * MAX_SOURCES)]


MAX_GROUPS = 4
MAX_GROUP_SOURCES = 16


class gpb_row_group(ctypes.Structure):
    _fields_ = [("d_staging", ctypes.c_void_p), ("n_staging_rows", ctypes.c_int64),
                ("d_cur_rows", ctypes.c_void_p), ("row_bytes", ctypes.c_int32)]


class gpb_gather_group(ctypes.Structure):
    _fields_ = [("d_dense", ctypes.c_void_p), ("table", ctypes.POINTER(gpb_sources)),
                ("row_bytes", ctypes.c_int32)]


class gpb_layer_group(ctypes.Structure):
    _fields_ = [("d_dense", ctypes.c_void_p), ("table", ctypes.POINTER(gpb_sources)),
                ("d_staging", ctypes.c_void_p), ("n_staging_rows", ctypes.c_int64),
                ("d_cur_rows", ctypes.c_void_p), ("row_bytes", ctypes.c_int32)]


def _hip_runtimes():
    """Distinct libamdhip64 files mapped into this process."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                path = line.split()[-1] if len(line.split()) >= 6 else ""
                if "libamdhip64" in os.path.basename(path):
                    found.add(os.path.realpath(path))
    except OSError:
        pass
    return found


def _load(path):
    if not os.path.exists(path):
        raise ImportError("libgpb.so not built at %s: run python "
                          "gather_plan_build_amd/build.py (no fallback exists)" % path)
    # torch provides device memory and streams; its HIP runtime must be the
    # one libgpb.so binds to (same SONAME, loaded first), or the process would
    # hold two runtimes whose streams and devices do not mix.
    import torch  # noqa: F401
    import torch.cuda  # noqa: F401
    lib = ctypes.CDLL(path)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded (%s): load torch before "
                          "libgpb.so" % ", ".join(sorted(runtimes)))
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.gpb_plan_sizes.argtypes = [ctypes.POINTER(gpb_batch), _I32P, _I32P, _I32P]
    lib.gpb_plan_build.argtypes = [ctypes.POINTER(gpb_batch), ctypes.POINTER(gpb_plan), vp]
    lib.gpb_plan_build_clear.argtypes = [ctypes.POINTER(gpb_batch), ctypes.POINTER(gpb_plan),
                                         vp, i64, vp]
    lib.gpb_writer_counts.argtypes = [ctypes.POINTER(gpb_batch), _I32P]
    lib.gpb_compose_gather_records.argtypes = [vp, ctypes.POINTER(gpb_sources), vp, i32, i32,
                                               i32, i32, vp, vp]
    lib.gpb_compose_layer.argtypes = [vp, ctypes.POINTER(gpb_sources),
                                      ctypes.POINTER(gpb_plan), i32, i32, vp, i64, vp, i32,
                                      i32, i32, vp, vp]
    lib.gpb_compose_consume.argtypes = lib.gpb_compose_layer.argtypes
    lib.gpb_compose_layer_noalloc.argtypes = [vp, ctypes.POINTER(gpb_sources), i32, i32,
                                              ctypes.POINTER(gpb_plan), i32, i32, vp, i32,
                                              i32, i32, vp, vp]
    lib.gpb_compose_layer_fill.argtypes = [vp, ctypes.POINTER(gpb_sources),
                                           ctypes.POINTER(gpb_plan), i32, i32, vp, i64, vp,
                                           i64, vp, i32, i32, i32, vp, vp]
    lib.gpb_compose_layer_ahead.argtypes = [vp] + list(lib.gpb_compose_layer.argtypes)
    lib.gpb_compose_consume_fill.argtypes = lib.gpb_compose_layer_fill.argtypes
    lib.gpb_compose_layer_ahead_fill.argtypes = [vp] + list(lib.gpb_compose_layer_fill.argtypes)
    lib.gpb_staging_clear.argtypes = [vp, i64, vp]
    lib.gpb_current_row_scatter.argtypes = [vp, i64, vp, vp, i32, i32, vp, vp]
    lib.gpb_compose_gather.argtypes = [vp, ctypes.POINTER(gpb_sources), vp, vp, i32,
                                       i32, i32, vp, vp]
    lib.gpb_compose_gather_slots.argtypes = [vp, ctypes.POINTER(gpb_sources), vp, i32, vp,
                                             vp, i32, i32, i32, vp, vp]
    lib.gpb_current_row_fill.argtypes = [vp, i64, vp, vp, i64, vp, vp, i32, i32, vp, vp]
    lib.gpb_current_row_scatter_groups.argtypes = [ctypes.POINTER(gpb_row_group), i32, vp,
                                                   i32, vp, vp]
    lib.gpb_compose_gather_groups.argtypes = [ctypes.POINTER(gpb_gather_group), i32, vp, vp,
                                              i32, i32, vp, vp]
    lib.gpb_compose_layer_groups.argtypes = [ctypes.POINTER(gpb_layer_group), i32,
                                             ctypes.POINTER(gpb_plan), i32, i32, i32, i32,
                                             vp, vp]
    lib.gpb_strerror.argtypes = [ctypes.c_int]
    lib.gpb_strerror.restype = ctypes.c_char_p
    for f in EXPORTS:
        if f != "gpb_strerror":
            getattr(lib, f).restype = ctypes.c_int
    return lib


EXPORTS = ("gpb_plan_sizes", "gpb_plan_build", "gpb_plan_build_clear",
           "gpb_writer_counts", "gpb_staging_clear", "gpb_current_row_scatter",
           "gpb_compose_gather", "gpb_compose_gather_slots", "gpb_compose_gather_records",
           "gpb_compose_layer", "gpb_compose_layer_fill", "gpb_compose_consume",
           "gpb_compose_layer_ahead", "gpb_compose_layer_noalloc",
           "gpb_compose_consume_fill", "gpb_compose_layer_ahead_fill",
           "gpb_current_row_fill", "gpb_current_row_scatter_groups",
           "gpb_compose_gather_groups", "gpb_compose_layer_groups", "gpb_strerror")

lib = _load(LIB_PATH)


class GpbError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__("%s: %s (%d)" % (what, strerror(code), code))


def strerror(code):
    return lib.gpb_strerror(int(code)).decode()


def _check(rc, what):
    if rc != OK:
        raise GpbError(rc, what)


def _ptr(x):
    """Device address of a GPU torch tensor, or an int address (taken as a
    device address), or None.  A tensor in host memory is refused: its address
    would reach a kernel."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("a %s tensor in host memory was passed where device memory "
                         "is required" % (tuple(x.shape),))
    return x.data_ptr()


def _gpu_device(device):
    import torch
    dev = torch.device(device)
    if dev.type != "cuda":
        raise ValueError("the compose runs on the GPU: device %s is not a GPU device" % dev)
    return dev


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _host_i32(a):
    """Contiguous int32 copy of host metadata; values outside int32 raise
    instead of wrapping."""
    v = np.asarray(a, dtype=np.int64).reshape(-1)
    if v.size and (v.min() < np.iinfo(np.int32).min or v.max() > np.iinfo(np.int32).max):
        raise ValueError("batch metadata value outside int32")
    return np.ascontiguousarray(v.astype(np.int32))


class BatchMeta:
    """Host side of a gpb_batch: geometry plus the three host arrays."""

    def __init__(self, bs, page_size, row_bytes, n_pool_pages, n_pool_entries,
                 n_writers, staging_cap_pages, prefix_pages, cur_tokens, req_pages):
        self.h_prefix = _host_i32(prefix_pages)
        self.h_cur = _host_i32(cur_tokens)
        self.h_req = _host_i32(req_pages)
        self.c = gpb_batch(bs, page_size, row_bytes, n_pool_pages, n_pool_entries,
                           n_writers, staging_cap_pages,
                           self.h_prefix.ctypes.data if self.h_prefix.size else None,
                           self.h_cur.ctypes.data if self.h_cur.size else None,
                           self.h_req.ctypes.data if self.h_req.size else None,
                           None, None, None)

    @classmethod
    def of(cls, b):
        """From any object with the workload attributes (workloads.Batch)."""
        return cls(b.bs, b.page_size, b.row_bytes, b.n_pool_pages, b.n_pool_entries,
                   b.n_writers, b.staging_cap_pages, b.prefix_pages, b.cur_tokens,
                   b.req_pages)

    def plan_key(self):
        """What a plan depends on (page 0d87bc5, commit "descriptor cache on
        the slot-remap objects": descriptors are cached for one batch and
        never reused across a different page layout, slot spans, table
        layout, device or capacity; page d63fbd4, commit "counting barrier +
        CUDA-IPC gather": the plan cache lives on the batch's slot remap): the
        geometry except the row size, and the three metadata arrays.  Two
        batches with equal keys have identical plans; the device is checked
        beside the key."""
        import hashlib
        c = self.c
        h = hashlib.sha256()
        for a in (self.h_prefix, self.h_cur, self.h_req):
            h.update(np.int64(a.size).tobytes())
            h.update(a.tobytes())
        return (c.bs, c.page_size, c.n_pool_pages, c.n_pool_entries, c.n_writers,
                c.staging_cap_pages, h.hexdigest())


def writer_counts(meta):
    """Entries of every writer's scatter list (host only, no device read)."""
    out = np.zeros(max(meta.c.n_writers, 1), np.int32)
    _check(lib.gpb_writer_counts(ctypes.byref(meta.c), out.ctypes.data_as(_I32P)),
           "gpb_writer_counts")
    return out[:meta.c.n_writers]


def plan_sizes(meta):
    """(S, T, NCP) after host validation; raises GpbError on a bad batch."""
    S, T, NCP = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib.gpb_plan_sizes(ctypes.byref(meta.c), ctypes.byref(S), ctypes.byref(T),
                              ctypes.byref(NCP)), "gpb_plan_sizes")
    return S.value, T.value, NCP.value


class Plan:
    """Device inputs and outputs of gpb_plan_build for one batch.

    Construction validates the batch on the host, copies the three metadata
    arrays to the device once and allocates every output (torch int32).
    ``build`` launches the plan kernels; the outputs are ``self.t[name]``."""

    def __init__(self, meta, device="cuda"):
        import torch
        self.meta = meta
        self.S, self.T, self.NCP = plan_sizes(meta)
        b = meta.c
        dev = _gpu_device(device)
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.key = meta.plan_key()
        self.d_prefix = torch.from_numpy(meta.h_prefix).to(dev)
        self.d_cur = torch.from_numpy(meta.h_cur).to(dev)
        self.d_req = torch.from_numpy(meta.h_req).to(dev)
        b.d_prefix_pages = self.d_prefix.data_ptr() if self.d_prefix.numel() else None
        b.d_cur_tokens = self.d_cur.data_ptr() if self.d_cur.numel() else None
        b.d_req_pages = self.d_req.data_ptr() if self.d_req.numel() else None
        bs, npp = b.bs, b.n_pool_pages
        sizes = {"slot_base": bs, "prefix_span": 2 * bs, "current_span": 2 * bs,
                 "q_lens": bs, "kv_lens": bs, "q_starts": bs, "k_bases": bs,
                 "q_bases": bs, "current_bases": bs, "slot_pages": self.S,
                 "owner": self.S, "src": self.S, "page_inverse": npp,
                 "staging_page_inverse": npp, "writer": self.NCP,
                 "staging_rows": self.T, "mixed_locs": self.T, "token_req": self.T,
                 "topk_offsets": self.T, "segments": 4 * bs,
                 "prefix_slots": self.S - self.NCP, "current_slots": self.NCP,
                 "pool_locs": self.T, "cur_page_token0": self.NCP,
                 "cur_page_ntok": self.NCP, "prefix_desc": 4 * (self.S - self.NCP),
                 "current_desc": 4 * self.NCP, "writer_offsets": b.n_writers + 1,
                 "writer_tokens": self.T, "writer_rows": self.T,
                 "writer_page_row0": self.NCP}
        self.t = {k: torch.empty(sizes[k], dtype=torch.int32, device=dev)
                  for k in PLAN_FIELDS}
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.c = gpb_plan(*[(self.t[k].data_ptr() if sizes[k] else None)
                            for k in PLAN_FIELDS], self.status.data_ptr())

    def build(self, stream=None, clear=None):
        """Launch the plan kernels; with ``clear`` (a uint8 device tensor) the
        same launches also zero it (gpb_plan_build_clear)."""
        if clear is None:
            _check(lib.gpb_plan_build(ctypes.byref(self.meta.c), ctypes.byref(self.c),
                                      _stream(stream)), "gpb_plan_build")
        else:
            _check(lib.gpb_plan_build_clear(ctypes.byref(self.meta.c), ctypes.byref(self.c),
                                            _ptr(clear), clear.numel() * clear.element_size(),
                                            _stream(stream)), "gpb_plan_build_clear")
        return self


def plan_build(meta, device="cuda", stream=None):
    """Validate, allocate and launch: returns the Plan (outputs in .t)."""
    return Plan(meta, device).build(stream)


class Sources:
    """A gpb_sources pointer table: [(base, n_pages), ...] with base a tensor
    or a device address.  Built once, passed by reference to every gather."""

    def __init__(self, entries):
        if not 1 <= len(entries) <= MAX_SOURCES:
            raise GpbError(EINVAL, "Sources")
        self.keep = [e[0] for e in entries]
        self.c = gpb_sources()
        self.c.n = len(entries)
        for i, (base, n_pages) in enumerate(entries):
            self.c.base[i] = _ptr(base)
            self.c.n_pages[i] = int(n_pages)


def staging_clear(buf, n_bytes=None, stream=None):
    """Zero a staging region (tensor, or address with n_bytes)."""
    if n_bytes is None:
        n_bytes = buf.numel() * buf.element_size()
    _check(lib.gpb_staging_clear(_ptr(buf), int(n_bytes), _stream(stream)),
           "gpb_staging_clear")


def current_row_scatter(staging, n_staging_rows, staging_rows, cur_rows, n_rows,
                        row_bytes, status=None, stream=None):
    _check(lib.gpb_current_row_scatter(_ptr(staging), int(n_staging_rows),
                                       _ptr(staging_rows), _ptr(cur_rows), int(n_rows),
                                       int(row_bytes), _ptr(status), _stream(stream)),
           "gpb_current_row_scatter")


def compose_gather(dense, sources, owner, src, n_slots, page_rows, row_bytes,
                   status=None, stream=None):
    if not isinstance(sources, Sources):
        sources = Sources(sources)
    _check(lib.gpb_compose_gather(_ptr(dense), ctypes.byref(sources.c), _ptr(owner),
                                  _ptr(src), int(n_slots), int(page_rows),
                                  int(row_bytes), _ptr(status), _stream(stream)),
           "gpb_compose_gather")


def compose_gather_slots(dense, sources, slots, n_list, owner, src, n_slots, page_rows,
                         row_bytes, status=None, stream=None):
    """Gather only the listed dense slots (prefetch or consume half)."""
    if not isinstance(sources, Sources):
        sources = Sources(sources)
    _check(lib.gpb_compose_gather_slots(_ptr(dense), ctypes.byref(sources.c), _ptr(slots),
                                        int(n_list), _ptr(owner), _ptr(src), int(n_slots),
                                        int(page_rows), int(row_bytes), _ptr(status),
                                        _stream(stream)),
           "gpb_compose_gather_slots")


def compose_gather_records(dense, sources, records, n_records, n_slots, page_rows,
                           row_bytes, status=None, stream=None):
    """Gather the pages named by (slot, owner, src, 0) records."""
    if not isinstance(sources, Sources):
        sources = Sources(sources)
    _check(lib.gpb_compose_gather_records(_ptr(dense), ctypes.byref(sources.c),
                                          _ptr(records), int(n_records), int(n_slots),
                                          int(page_rows), int(row_bytes), _ptr(status),
                                          _stream(stream)),
           "gpb_compose_gather_records")


def compose_layer(dense, sources, plan, n_slots, n_cur_pages, staging, n_staging_rows,
                  cur_rows, n_rows, page_rows, row_bytes, status=None, stream=None):
    """Scatter and gather of one layer in one launch (``plan`` a Plan)."""
    if not isinstance(sources, Sources):
        sources = Sources(sources)
    _check(lib.gpb_compose_layer(_ptr(dense), ctypes.byref(sources.c), ctypes.byref(plan.c),
                                 int(n_slots), int(n_cur_pages), _ptr(staging),
                                 int(n_staging_rows), _ptr(cur_rows), int(n_rows),
                                 int(page_rows), int(row_bytes), _ptr(status),
                                 _stream(stream)),
           "gpb_compose_layer")


def compose_layer_noalloc(dense, pools, n_writers, staging_cap_pages, plan, n_slots,
                          n_cur_pages, cur_rows, n_rows, page_rows, row_bytes, status=None,
                          stream=None):
    """The one-launch layer with staging in the library's static array:
    ``pools`` lists the pool entries only, the library adds the slabs."""
    if not isinstance(pools, Sources):
        pools = Sources(pools)
    _check(lib.gpb_compose_layer_noalloc(_ptr(dense), ctypes.byref(pools.c), int(n_writers),
                                         int(staging_cap_pages), ctypes.byref(plan.c),
                                         int(n_slots), int(n_cur_pages), _ptr(cur_rows),
                                         int(n_rows), int(page_rows), int(row_bytes),
                                         _ptr(status), _stream(stream)),
           "gpb_compose_layer_noalloc")


def compose_layer_fill(dense, sources, plan, n_slots, n_cur_pages, staging, n_staging_rows,
                       pool, n_pool_rows, cur_rows, n_rows, page_rows, row_bytes, status=None,
                       stream=None):
    """The one-launch layer with the fused fill (current rows also to their
    pool rows)."""
    if not isinstance(sources, Sources):
        sources = Sources(sources)
    _check(lib.gpb_compose_layer_fill(_ptr(dense), ctypes.byref(sources.c),
                                      ctypes.byref(plan.c), int(n_slots), int(n_cur_pages),
                                      _ptr(staging), int(n_staging_rows), _ptr(pool),
                                      int(n_pool_rows), _ptr(cur_rows), int(n_rows),
                                      int(page_rows), int(row_bytes), _ptr(status),
                                      _stream(stream)),
           "gpb_compose_layer_fill")


def compose_consume(dense, sources, plan, n_slots, n_cur_pages, staging, n_staging_rows,
                    cur_rows, n_rows, page_rows, row_bytes, status=None, stream=None):
    """The consume half in one launch: scatter and current-page gather."""
    if not isinstance(sources, Sources):
        sources = Sources(sources)
    _check(lib.gpb_compose_consume(_ptr(dense), ctypes.byref(sources.c), ctypes.byref(plan.c),
                                   int(n_slots), int(n_cur_pages), _ptr(staging),
                                   int(n_staging_rows), _ptr(cur_rows), int(n_rows),
                                   int(page_rows), int(row_bytes), _ptr(status),
                                   _stream(stream)),
           "gpb_compose_consume")


def compose_layer_ahead(dense, dense_next, sources, plan, n_slots, n_cur_pages, staging,
                        n_staging_rows, cur_rows, n_rows, page_rows, row_bytes, status=None,
                        stream=None):
    """This layer's consume and the next layer's prefix pages in one launch."""
    if not isinstance(sources, Sources):
        sources = Sources(sources)
    _check(lib.gpb_compose_layer_ahead(_ptr(dense), _ptr(dense_next), ctypes.byref(sources.c),
                                       ctypes.byref(plan.c), int(n_slots), int(n_cur_pages),
                                       _ptr(staging), int(n_staging_rows), _ptr(cur_rows),
                                       int(n_rows), int(page_rows), int(row_bytes),
                                       _ptr(status), _stream(stream)),
           "gpb_compose_layer_ahead")


def compose_consume_fill(dense, sources, plan, n_slots, n_cur_pages, staging, n_staging_rows,
                         pool, n_pool_rows, cur_rows, n_rows, page_rows, row_bytes, status=None,
                         stream=None):
    """The consume half in one launch with the fused fill (current rows also
    to their pool rows)."""
    if not isinstance(sources, Sources):
        sources = Sources(sources)
    _check(lib.gpb_compose_consume_fill(_ptr(dense), ctypes.byref(sources.c),
                                        ctypes.byref(plan.c), int(n_slots), int(n_cur_pages),
                                        _ptr(staging), int(n_staging_rows), _ptr(pool),
                                        int(n_pool_rows), _ptr(cur_rows), int(n_rows),
                                        int(page_rows), int(row_bytes), _ptr(status),
                                        _stream(stream)),
           "gpb_compose_consume_fill")


def compose_layer_ahead_fill(dense, dense_next, sources, plan, n_slots, n_cur_pages, staging,
                             n_staging_rows, pool, n_pool_rows, cur_rows, n_rows, page_rows,
                             row_bytes, status=None, stream=None):
    """This layer's consume with the fused fill and the next layer's prefix
    pages in one launch."""
    if not isinstance(sources, Sources):
        sources = Sources(sources)
    _check(lib.gpb_compose_layer_ahead_fill(_ptr(dense), _ptr(dense_next),
                                            ctypes.byref(sources.c), ctypes.byref(plan.c),
                                            int(n_slots), int(n_cur_pages), _ptr(staging),
                                            int(n_staging_rows), _ptr(pool), int(n_pool_rows),
                                            _ptr(cur_rows), int(n_rows), int(page_rows),
                                            int(row_bytes), _ptr(status), _stream(stream)),
           "gpb_compose_layer_ahead_fill")


def current_row_fill(staging, n_staging_rows, staging_rows, pool, n_pool_rows, pool_locs,
                     cur_rows, n_rows, row_bytes, status=None, stream=None):
    """Each current row to its staging row and to its pool row, one pass."""
    _check(lib.gpb_current_row_fill(_ptr(staging), int(n_staging_rows), _ptr(staging_rows),
                                    _ptr(pool), int(n_pool_rows), _ptr(pool_locs),
                                    _ptr(cur_rows), int(n_rows), int(row_bytes),
                                    _ptr(status), _stream(stream)),
           "gpb_current_row_fill")


def current_row_scatter_groups(groups, staging_rows, n_rows, status=None, stream=None):
    """One launch scattering the current rows of every group:
    groups = [(staging, n_staging_rows, cur_rows, row_bytes), ...]."""
    arr = (gpb_row_group * max(len(groups), 1))(
        *[gpb_row_group(_ptr(st), int(n), _ptr(cur), int(rb)) for st, n, cur, rb in groups])
    _check(lib.gpb_current_row_scatter_groups(arr, len(groups), _ptr(staging_rows),
                                              int(n_rows), _ptr(status), _stream(stream)),
           "gpb_current_row_scatter_groups")


def compose_gather_groups(groups, owner, src, n_slots, page_rows, status=None, stream=None):
    """One launch gathering every group: groups = [(dense, Sources, row_bytes), ...]."""
    keep = [g[1] if isinstance(g[1], Sources) else Sources(g[1]) for g in groups]
    arr = (gpb_gather_group * max(len(groups), 1))(
        *[gpb_gather_group(_ptr(d), ctypes.pointer(t.c), int(rb))
          for (d, _, rb), t in zip(groups, keep)])
    _check(lib.gpb_compose_gather_groups(arr, len(groups), _ptr(owner), _ptr(src),
                                         int(n_slots), int(page_rows), _ptr(status),
                                         _stream(stream)),
           "gpb_compose_gather_groups")


def compose_layer_groups(groups, plan, n_slots, n_cur_pages, n_rows, page_rows, status=None,
                         stream=None):
    """One launch composing one layer of every group: groups = [(dense, Sources, staging,
    n_staging_rows, cur_rows, row_bytes), ...] on one plan (a Plan)."""
    keep = [g[1] if isinstance(g[1], Sources) else Sources(g[1]) for g in groups]
    arr = (gpb_layer_group * max(len(groups), 1))(
        *[gpb_layer_group(_ptr(d), ctypes.pointer(t.c), _ptr(st), int(n), _ptr(cur), int(rb))
          for (d, _, st, n, cur, rb), t in zip(groups, keep)])
    _check(lib.gpb_compose_layer_groups(arr, len(groups), ctypes.byref(plan.c), int(n_slots),
                                        int(n_cur_pages), int(n_rows), int(page_rows),
                                        _ptr(status), _stream(stream)),
           "gpb_compose_layer_groups")
