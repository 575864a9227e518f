"""Benchmark of the KV-compose hot path on one MI355X.

One step = one batch through the whole path: plan build, staging clear, then
for each of the 78 layers the current-row scatter and the slot-dense page
gather (traced workload: bs=12, 44,600 current tokens split by Dirichlet(1),
prefix 0-32K tokens per request, 64-token pages, 1152-byte rows = 576 bf16,
pools rotated over 4 arenas so no layer's reads fit the 256 MB MALL).
Inputs are resident in HBM before timing starts.

Prints one JSON line.  ``value`` is the whole job's algorithmic HBM
throughput of the compose (bytes the method must move per layer -- read and
write every dense page and every current row, plus descriptors -- times 78
layers, over the measured step time; the step also holds the plan build and
staging clear, whose bytes are not counted).  The timed region holds the K
steps and nothing else.  Per-kernel average durations come from regions of
back-to-back launches of one kernel with the layer loop's arguments (HIP
events on the launch stream around each region): events between kernels
would add their own cache flushes to what they measure.  ``cpu_baseline``
times the CPU oracle on a bounded sample of the same layers on this host.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
METRIC = ("compose µs/layer and achieved HBM GB/s (% of peak) at bs=12, "
          "44.6K current tokens")


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 1000 traced steps are about 7 s of timed GPU work
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="traced",
                    choices=["traced", "opaque", "medium", "multi_source", "tiny"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget for the CPU oracle sample (0 disables it)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE", "FETCH", "WRITE"),
                    help="write profiles/ summaries from three rocprofv3 csv output "
                         "directories (kernel trace + stats, FETCH_SIZE, WRITE_SIZE) "
                         "and exit; runs on the host only")
    ap.add_argument("--summarize-trace", metavar="TRACE",
                    help="write profiles/compose_<workload>_kernels.txt from a rocprofv3 "
                         "kernel-trace directory alone (no counter passes) and exit")
    ap.add_argument("--summarize-extras", metavar="TRACE",
                    help="write profiles/compose_<workload>_extras_kernels.txt from the "
                         "rocprofv3 kernel-trace directory of a default run and exit")
    ap.add_argument("--summarize-extras-counters", nargs=2, metavar=("FETCH", "WRITE"),
                    help="write profiles/compose_<workload>_extras_counters.txt from the "
                         "FETCH_SIZE and WRITE_SIZE runs of a default run with the extras "
                         "and exit")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the headline path only (no prefetch split, fused fill "
                         "or twin): the mode the profiler runs use")
    ap.add_argument("--twin-index-bytes", type=int, default=144,
                    help="also time the indexer-key twin compose with rows of this "
                         "many bytes on the same plan (0 disables it)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="end with three torch copies of this size (counter "
                         "calibration under rocprofv3)")
    return ap.parse_args()


# The library whose kernels the counters were taken on (GPB_LIB overrides
# the in-tree build, as it does for the binding).
LIB = os.environ.get("GPB_LIB", os.path.join(ROOT, "gather_plan_build_amd", "libgpb.so"))
_BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _elf_section(data, name):
    """Bytes of the named section of a 64-bit little-endian ELF image."""
    import struct
    shoff = struct.unpack_from("<Q", data, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    heads = [struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize)
             for i in range(shnum)]
    names = heads[shstrndx][4]
    for h in heads:
        at = names + h[0]
        if data[at:data.index(b"\0", at)].decode() == name:
            return data[h[4]:h[4] + h[5]]
    return None


def _kernel_digest(lib=None):
    """Digest of the machine code of the library's gfx950 kernels: the .text
    of every gfx950 code object in its offload bundles.  It changes when a
    kernel's code does and not when only host code or comments do, so the
    counters stay attached to the kernels they were taken on."""
    import struct
    with open(lib or LIB, "rb") as f:
        data = f.read()
    fatbin = _elf_section(data, ".hip_fatbin") or b""
    h = hashlib.sha256()
    at = fatbin.find(_BUNDLE_MAGIC)
    while at >= 0:
        n = struct.unpack_from("<Q", fatbin, at + len(_BUNDLE_MAGIC))[0]
        q = at + len(_BUNDLE_MAGIC) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, q)
            triple = fatbin[q + 24:q + 24 + tlen].decode()
            q += 24 + tlen
            if triple.endswith("gfx950"):
                h.update(_elf_section(fatbin[at + off:at + off + size], ".text") or b"")
        at = fatbin.find(_BUNDLE_MAGIC, at + len(_BUNDLE_MAGIC))
    return h.hexdigest()[:16]


def _traffic(workload):
    """Memory bytes per one-launch-layer launch from the committed rocprofv3
    counter summary, if it was taken on the kernels the library now holds."""
    path = os.path.join(ROOT, "profiles", "compose_layer_%s_counters.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_digest") != _kernel_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def _host_threads():
    """Worker threads for the parallel oracle leg: the cores this process may
    run on, at most 16 (one GPU's share of a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(batch, pools, curs, budget_s, threads=None):
    """The CPU oracle (plain C loops) on the same batch, the plan built once:

    - headline: layers on one thread until the budget is spent (median per
      layer);
    - "threaded": one layer at a time on ``threads`` threads, split as
      contiguous slot ranges: the staging zero and the row scatter on one
      thread (the oracle's layer with no slots), then the gather as one
      contiguous range of dense slots per thread (the oracle's slot-list
      gather), a quarter of the budget;
    - "concurrent_layers": ``threads`` copies of the single-threaded oracle
      running different layers at once, each with its own staging and dense
      buffers, a quarter of the budget (host throughput, not latency).

    The oracle itself is the same in all three; only how its calls are spread
    over threads differs."""
    import threading
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle
    orc = oracle.default()
    t0 = time.perf_counter()
    want = oracle.plan_for(batch, orc)
    plan_s = time.perf_counter() - t0
    host_pools, host_curs = {}, {}
    for k in range(min(len(pools), batch.n_layers)):
        host_pools[k] = pools[k].cpu().numpy().reshape(-1)
        host_curs[k] = curs[k].cpu().numpy()
    PS, RB = batch.page_size, batch.row_bytes

    def run_layer(layer, staging):
        k = layer % len(pools)
        return oracle.layer_for(batch, want, host_pools[k], host_curs[k], staging, orc)

    staging = np.empty(batch.staging_rows_total * RB, np.uint8)
    per_layer = []
    spent = 0.0
    runs = 0
    # cycle through the batch's layers until the budget is spent (at least
    # one pass over every layer)
    while spent < budget_s or runs < batch.n_layers:
        t0 = time.perf_counter()
        run_layer(runs % batch.n_layers, staging)
        dt = time.perf_counter() - t0
        per_layer.append(dt)
        spent += dt
        runs += 1
    S, T = batch.n_req_pages, batch.n_cur_tokens
    layer_bytes = (2 * S * PS * RB + 2 * T * RB + 8 * S + 4 * T
                   + 8 * (batch.n_pool_entries + batch.n_writers))
    med = sorted(per_layer)[len(per_layer) // 2]
    out = {"value": round(layer_bytes / med / 1e9, 3), "unit": "GB/s", "cores": 1,
           "kind": "oracle",
           "us_per_layer": round(med * 1e6, 1),
           "plan_us": round(plan_s * 1e6, 1),
           "sample": "%d layer runs (the %s workload's %d layers, cycled; %.1f s of "
                     "CPU work; median per layer; plan once), single-threaded C "
                     "oracle: zero staging, scatter current rows, gather every page"
                     % (runs, batch.name, batch.n_layers, spent),
           "cpu_model": _cpu_model(), "host_threads_available": os.cpu_count()}

    n = threads if threads is not None else _host_threads()
    if n <= 1:
        return out

    # one layer on n threads, split by contiguous slot ranges
    bounds = np.linspace(0, S, n + 1).astype(np.int64)
    ranges = [np.arange(bounds[i], bounds[i + 1], dtype=np.int32) for i in range(n)]
    dense = np.empty((S * PS, RB), np.uint8)
    no_slots = want["owner"][:0]

    def split_layer(pool_exec, layer):
        k = layer % len(pools)
        table = oracle.pointer_table(host_pools[k], staging, batch.n_pool_entries,
                                     batch.n_writers, batch.staging_cap_pages, PS, RB)
        orc.compose_layer(table, host_curs[k], want["staging_rows"], no_slots, no_slots,
                          PS, RB, staging)  # staging zero + scatter only
        list(pool_exec.map(lambda sl: orc.gather_slots(table, sl, want["owner"], want["src"],
                                                       PS, RB, dense), ranges))

    with ThreadPoolExecutor(n) as ex:
        split_layer(ex, 0)  # untimed: first touch; also checked against the one-thread layer
        ref, _ = run_layer(0, np.empty_like(staging))
        if not np.array_equal(ref, dense):
            raise AssertionError("slot-range split of the oracle differs from the oracle")
        del ref
        split = []
        spent = 0.0
        while spent < budget_s / 4 or len(split) < 3:
            t0 = time.perf_counter()
            split_layer(ex, len(split) % batch.n_layers)
            dt = time.perf_counter() - t0
            split.append(dt)
            spent += dt
    med_split = sorted(split)[len(split) // 2]
    out["threaded"] = {
        "value": round(layer_bytes / med_split / 1e9, 3), "unit": "GB/s", "cores": n,
        "kind": "oracle", "us_per_layer": round(med_split * 1e6, 1),
        "sample": "%d layer runs, median per layer; staging zero and row scatter on one "
                  "thread, then the gather as %d contiguous slot ranges on %d threads"
                  % (len(split), n, n)}
    del dense

    # n single-threaded oracles on different layers at once
    done = [0] * n
    seconds = max(budget_s / 4, 1e-3)
    barrier = threading.Barrier(n + 1)

    def worker(w):
        st = np.empty(batch.staging_rows_total * RB, np.uint8)
        run_layer(w % batch.n_layers, st)  # untimed: first touch of its buffers
        barrier.wait()
        deadline = time.perf_counter() + seconds
        layer = w
        while time.perf_counter() < deadline:
            run_layer(layer % batch.n_layers, st)
            done[w] += 1
            layer += n

    # the oracle's C calls release the GIL (ctypes), so the copies run
    # concurrently; all start together and run for the same wall time
    workers = [threading.Thread(target=worker, args=(w,)) for w in range(n)]
    for t in workers:
        t.start()
    barrier.wait()
    t0 = time.perf_counter()
    for t in workers:
        t.join()
    wall = time.perf_counter() - t0
    total = sum(done)
    out["concurrent_layers"] = {
        "value": round(layer_bytes * total / wall / 1e9, 3), "unit": "GB/s",
        "cores": n, "kind": "oracle",
        "sample": "%d layer runs over %.1f s wall on %d threads, each a copy of "
                  "the single-threaded oracle with its own staging and dense "
                  "buffers" % (total, wall, n)}
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _csv_rows(directory, suffix):
    import csv
    import glob
    out = []
    for path in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix),
                                 recursive=True)):
        with open(path, newline="") as f:
            out += list(csv.DictReader(f))
    return out


def _short(name):
    """Kernel name without namespaces and parameter list; template arguments
    kept (they tell the gather from the slot-list gather, the scatter from the
    fused fill)."""
    import re
    for key in ("k_compose_layer_fill", "k_compose_layer", "k_layer_groups", "k_compose_gather", "k_row_scatter",
                "k_gather_groups",
                "k_scatter_groups", "k_fill_zero", "k_plan_scan_fill", "k_plan_slots",
                "k_plan_tokens", "copyBuffer"):
        if key in name:
            m = re.search(key + r"(<[^>]*>)?", name)
            return m.group(0).replace(" ", "")
    return name[:60]


# $REPO is the repository root, $OUT the directory the runs write to
EXTRAS_TRACE_COMMAND = (
    "cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format csv "
    "-d $OUT/prof_extras -o extras -- python3 $REPO/bench.py "
    "--steps 2 --warmup 1 --cpu-seconds 0")

ONE_LAYER_WORKLOADS = ("medium", "multi_source", "tiny")

PROFILE_COMMANDS = {
    "trace": "cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format csv "
             "-d $OUT/prof_trace -o trace -- python3 $REPO/bench.py "
             "--steps 3 --warmup 1 --cpu-seconds 0 --no-extras",
    "fetch": "cd /tmp && TMPDIR=/tmp rocprofv3 --pmc FETCH_SIZE --output-format csv "
             "-d $OUT/prof_fetch -o fetch -- python3 $REPO/bench.py "
             "--steps 1 --warmup 0 --cpu-seconds 0 --no-extras --calibration-copy-mib 1024",
    "write": "cd /tmp && TMPDIR=/tmp rocprofv3 --pmc WRITE_SIZE --output-format csv "
             "-d $OUT/prof_write -o write -- python3 $REPO/bench.py "
             "--steps 1 --warmup 0 --cpu-seconds 0 --no-extras --calibration-copy-mib 1024",
    "summary": "python3 bench.py --summarize-profiles $OUT/prof_trace "
               "$OUT/prof_fetch $OUT/prof_write",
}


def _profile_commands(trace_dir, workload="traced"):
    """PROFILE_COMMANDS with $OUT set to the directory the runs wrote to, for
    the given workload."""
    out = os.path.relpath(os.path.dirname(os.path.abspath(trace_dir)), ROOT)
    flag = "" if workload == "traced" else " --workload " + workload
    cmds = {}
    for k, v in PROFILE_COMMANDS.items():
        v = v.replace("$OUT", "$REPO/" + out if k != "summary" else out)
        if k == "trace" and workload in ONE_LAYER_WORKLOADS:
            # one layer per step: more steps, so every kernel has enough calls
            v = v.replace("--steps 3 ", "--steps 50 ")
        cmds[k] = (v + flag) if k == "summary" else v.replace("bench.py", "bench.py" + flag, 1)
    return cmds


def summarize_extras(trace_dir, workload="traced"):
    """profiles/compose_<workload>_extras_kernels.txt: kernel statistics of a
    default bench run (headline path plus the prefetch split, fused fill,
    index-key twin and grouped launches), trace only."""
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    out = os.path.relpath(os.path.dirname(os.path.abspath(trace_dir)), ROOT)
    cmd = EXTRAS_TRACE_COMMAND.replace("$OUT", "$REPO/" + out)
    if workload != "traced":
        cmd = cmd.replace("bench.py", "bench.py --workload " + workload, 1)
    lines = ["# rocprofv3 kernel statistics, %s workload with the extras "
             "(bench.py default run)" % workload,
             "# command: " + cmd,
             "# k_compose_gather<64,1,M>: M = 0 all slots, 1 slot list, 2 records (split "
             "halves); k_row_scatter<64,1,FILL,SROWS>: FILL = fused fill; "
             "k_compose_layer<64,SROWS>: one-launch layer, consume and layer-ahead launches; "
             "k_compose_layer_fill<64,SROWS>: the one-launch layer with the fused fill; "
             "*_groups = token KV and index twin in one launch",
             "%-34s %7s %12s %12s %12s %8s" % ("kernel", "calls", "avg_ns", "min_ns",
                                              "max_ns", "pct")]
    for r in stats:
        lines.append("%-34s %7s %12.0f %12.0f %12.0f %8.2f" % (
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]), float(r["MinNs"]),
            float(r["MaxNs"]), float(r["Percentage"])))
    path = os.path.join(ROOT, "profiles", "compose_%s_extras_kernels.txt" % workload)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


EXTRAS_COUNTER_COMMAND = (
    "cd /tmp && TMPDIR=/tmp rocprofv3 --pmc {counter} --output-format csv "
    "-d $OUT/prof_extras_{what} -o {what} -- python3 $REPO/bench.py "
    "--steps 1 --warmup 0 --cpu-seconds 0 --calibration-copy-mib 1024")


def summarize_extras_counters(fetch_dir, write_dir, workload="traced"):
    """profiles/compose_<workload>_extras_counters.txt: bytes per dispatch
    below L2 of every library kernel in a default run with the extras, per
    kernel and grid size (one launch shape per line: the one-launch layer,
    the consume alone, the record halves, ...), from FETCH_SIZE and
    WRITE_SIZE, each scaled by what it reads for a 1 GiB copy in the same
    run."""
    import re

    def per_shape(directory, counter):
        acc = {}
        for r in _csv_rows(directory, "counter_collection.csv"):
            if r.get("Counter_Name") != counter:
                continue
            m = re.search(r"(k_\w+(<[^>]*>)?|copyBuffer)", r["Kernel_Name"])
            name = m.group(0).replace(" ", "") if m else r["Kernel_Name"][:40]
            acc.setdefault((name, int(r.get("Grid_Size") or 0)), []).append(
                float(r["Counter_Value"]))
        return acc

    fetch, write = per_shape(fetch_dir, "FETCH_SIZE"), per_shape(write_dir, "WRITE_SIZE")
    copy_kib = 1024 * 1024.0
    f_scale = copy_kib / max(v for (k, g), vs in fetch.items() if k == "copyBuffer" for v in vs)
    w_scale = copy_kib / max(v for (k, g), vs in write.items() if k == "copyBuffer" for v in vs)
    out = os.path.relpath(os.path.dirname(os.path.abspath(fetch_dir)), ROOT)
    flag = "" if workload == "traced" else " --workload " + workload
    lines = ["# rocprofv3 counters below L2 per dispatch, %s workload, default run with "
             "the extras; FETCH_SIZE scaled by %.4f and WRITE_SIZE by %.4f (what each reads "
             "for a 1 GiB copy in the same run)" % (workload, f_scale, w_scale)]
    for what, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        cmd = EXTRAS_COUNTER_COMMAND.format(counter=counter, what=what)
        lines.append("# command: " + cmd.replace("$OUT", "$REPO/" + out)
                     .replace("bench.py", "bench.py" + flag, 1))
    lines.append("# kernel code digest of libgpb.so: %s" % _kernel_digest())
    lines.append("%-34s %10s %6s %14s %14s" % ("kernel", "workgroups", "calls", "read_MB",
                                               "write_MB"))
    for key in sorted(set(fetch) & set(write)):
        name, grid = key
        if not name.startswith("k_"):
            continue
        fk = sum(fetch[key]) / len(fetch[key])
        wk = sum(write[key]) / len(write[key])
        lines.append("%-34s %10d %6d %14.1f %14.1f" % (
            name, grid // 64 if "plan" not in name and "fill_zero" not in name else grid // 256,
            len(fetch[key]), fk * f_scale * 1024 / 1e6, wk * w_scale * 1024 / 1e6))
    path = os.path.join(ROOT, "profiles", "compose_%s_extras_counters.txt" % workload)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _kernel_table(trace_dir, workload, title):
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    lines = ["# rocprofv3 kernel statistics, %s workload (%s)" % (workload, title),
             "# command: " + _profile_commands(trace_dir, workload)["trace"],
             "# kernel code digest of libgpb.so (.text of its gfx950 code objects): %s"
             % _kernel_digest(),
             "%-34s %7s %12s %12s %12s %8s" % ("kernel", "calls", "avg_ns", "min_ns",
                                              "max_ns", "pct")]
    for r in stats:
        lines.append("%-34s %7s %12.0f %12.0f %12.0f %8.2f" % (
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]), float(r["MinNs"]),
            float(r["MaxNs"]), float(r["Percentage"])))
    return lines


def summarize_trace(trace_dir, workload="traced"):
    """profiles/compose_<workload>_kernels.txt from a kernel trace alone."""
    lines = _kernel_table(trace_dir, workload, "bench.py, kernel trace only")
    path = os.path.join(ROOT, "profiles", "compose_%s_kernels.txt" % workload)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_profiles(trace_dir, fetch_dir, write_dir, workload="traced"):
    """profiles/compose_<workload>_kernels.txt (rocprofv3 kernel statistics)
    and profiles/compose_layer_<workload>_counters.json (bytes per launch of
    every library kernel from FETCH_SIZE / WRITE_SIZE, each scaled by what
    the same counter reads for a plain 1 GiB copy; the one-launch layer's
    figure is the roofline's traffic)."""
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    lines = _kernel_table(trace_dir, workload, "bench.py")
    with open(os.path.join(prof, "compose_%s_kernels.txt" % workload), "w") as f:
        f.write("\n".join(lines) + "\n")

    def per_kernel(directory, counter):
        acc = {}
        for r in _csv_rows(directory, "counter_collection.csv"):
            if r.get("Counter_Name") != counter:
                continue
            acc.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return acc

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    # the calibration copies are the largest copyBuffer dispatches (1 GiB each;
    # the other copies are the 64 MiB input-generation chunks)
    copy_kib = 1024 * 1024.0
    f_copy, w_copy = max(fetch["copyBuffer"]), max(write["copyBuffer"])
    f_scale, w_scale = copy_kib / f_copy, copy_kib / w_copy
    rec = {"workload": workload, "kernel_digest": _kernel_digest(),
           "commands": _profile_commands(trace_dir, workload),
           "calibration": {"copy_bytes": int(copy_kib * 1024), "fetch_kib": f_copy,
                           "write_kib": w_copy, "fetch_scale": f_scale,
                           "write_scale": w_scale},
           "kernels": {}}
    for k in sorted(set(fetch) & set(write)):
        if not k.startswith("k_"):
            continue
        if k in fetch and k in write:
            fk = sum(fetch[k]) / len(fetch[k])
            wk = sum(write[k]) / len(write[k])
            rec["kernels"][k] = {
                "dispatches": len(fetch[k]), "fetch_kib_raw": round(fk, 1),
                "write_kib_raw": round(wk, 1),
                "read_bytes": round(1024 * fk * f_scale),
                "write_bytes": round(1024 * wk * w_scale),
                "hbm_bytes_per_launch": round(1024 * (fk * f_scale + wk * w_scale))}
    layer = [k for k in rec["kernels"] if k.startswith("k_compose_layer")]
    if layer:
        rec["kernel"] = layer[0]
        rec["hbm_bytes_per_launch"] = rec["kernels"][layer[0]]["hbm_bytes_per_launch"]
    with open(os.path.join(prof, "compose_layer_%s_counters.json" % workload), "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec, indent=1, sort_keys=True))
    return rec


class Lead:
    """GPU work queued ahead of a timed region: copies of a 256 MiB buffer,
    enough of them that the host has enqueued every call of the region
    before the GPU reaches the region's start event (HOST_US_PER_CALL per
    call, a generous bound on one ctypes call and its launches, plus a
    margin).  The region then holds GPU time only, even for calls whose host
    side is slower than their kernels (every call of a one-layer batch)."""
    HOST_US_PER_CALL = 30.0

    def __init__(self, stream):
        import torch
        n = 256 << 20
        self.src = torch.ones(n, dtype=torch.uint8, device="cuda")
        self.dst = torch.empty_like(self.src)
        self.copy_ms = _timed(stream, lambda: self.dst.copy_(self.src), 8)

    def __call__(self, n_calls):
        import math
        want_ms = n_calls * self.HOST_US_PER_CALL * 1e-3 + 0.5
        k = max(2, math.ceil(want_ms / self.copy_ms))
        return lambda: [self.dst.copy_(self.src) for _ in range(k)]


def _timed(stream, fn, reps, lead=None):
    """Average ms of ``fn`` over ``reps`` back-to-back calls, HIP events on
    the launch stream around the whole region.  ``lead`` enqueues GPU work
    before the start event, long enough that the host has queued every call
    before the GPU reaches it: the region then holds GPU time only, even for
    calls whose host side is slower than their kernels."""
    import torch
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if lead is not None:
        lead()
    start.record(stream)
    for _ in range(reps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / reps


def main():
    a = _args()
    if a.summarize_profiles:
        summarize_profiles(*a.summarize_profiles, workload=a.workload)
        return
    if a.summarize_trace:
        summarize_trace(a.summarize_trace, workload=a.workload)
        return
    if a.summarize_extras_counters:
        summarize_extras_counters(*a.summarize_extras_counters, workload=a.workload)
        return
    if a.summarize_extras:
        summarize_extras(a.summarize_extras, workload=a.workload)
        return
    if a.gpus != 1:
        print("bench.py measures one GPU only: the compose path here has no "
              "multi-GPU transport (the pointer table would hold peer addresses); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    sys.path.insert(0, ROOT)
    import gather_plan_build_amd as gpb
    import workloads

    batch = workloads.make_batch(a.workload)
    pools, curs = workloads.make_values(batch, device="cuda")
    runner = gpb.ComposeRunner(gpb.BatchMeta.of(batch), pools, curs)
    L = batch.n_layers
    stream = torch.cuda.current_stream()

    def step():
        runner.run(L, stream)

    for _ in range(a.warmup):
        step()
    # the timed region: K whole steps, nothing else on the stream
    ms_per_step = _timed(stream, step, a.steps)
    assert int(runner.status.item()) == 0, "a kernel flagged a bad descriptor or row"
    assert int(runner.plan.status.item()) == 0, "the plan kernels flagged their input"

    layer_bytes = runner.algorithmic_bytes_per_layer()
    value_gbs = layer_bytes * L / (ms_per_step * 1e-3) / 1e9
    lead = Lead(stream)
    # the median of single steps, each in a region of its own behind a lead
    # (a step of a one-layer batch is shorter than its host calls)
    one_ms = sorted(_timed(stream, step, 1, lead=lead(L + 3)) for _ in range(MEDIAN_STEPS))
    median_ms = 0.5 * (one_ms[(MEDIAN_STEPS - 1) // 2] + one_ms[MEDIAN_STEPS // 2])
    out = {"metric": METRIC, "value": round(value_gbs, 1), "unit": "GB/s",
           "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
           "ms_per_step": round(ms_per_step, 4),
           "ms_per_step_median": round(median_ms, 4), "median_of_steps": MEDIAN_STEPS,
           "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
           "config": {"workload": "%s: bs=%d, %d current tokens, %d dense slots, "
                                  "%d-token pages, %d-byte rows, %d layers, plan once "
                                  "per batch" % (batch.name, batch.bs, batch.n_cur_tokens,
                                                 batch.n_req_pages, batch.page_size,
                                                 batch.row_bytes, L),
                      "global_batch": batch.bs, "seq_len": None,
                      "parallelism": "single GPU",
                      "algorithmic_bytes_per_layer": layer_bytes}}
    # GPU-only regions, each behind a lead (see Lead): K*L back-to-back
    # layers, and each kernel alone with the layer loop's arguments; a batch
    # of few layers repeats its loop until a region holds at least
    # MIN_REGION_LAYERS layers, so a region of microsecond launches is not
    # a handful of calls
    reps = max(min(a.steps, MAX_REGION_REPS), -(-MIN_REGION_LAYERS // L))

    def region(fn, calls_per_rep):
        return _timed(stream, fn, reps, lead=lead(reps * calls_per_rep))

    layer_ms = region(lambda: [runner.layer(l, stream) for l in range(L)], L) / L
    two_ms = region(lambda: [runner.layer_two_launch(l, stream) for l in range(L)],
                    2 * L) / L
    g_ms = region(lambda: [runner.gather(l, stream) for l in range(L)], L) / L
    s_ms = region(lambda: [runner.scatter(l, stream) for l in range(L)], L) / L
    # plan build with the staging clear: three launches per batch; and the
    # plan build alone (gpb_plan_build, the same three launches, no clear)
    p_ms = region(lambda: runner.begin_batch(stream), 1)
    p0_ms = region(lambda: runner.plan.build(stream), 1)
    # host time of one gpb_plan_build_clear call (validation + three
    # launches, no synchronisation), for comparison with host-side builders
    torch.cuda.synchronize()
    n_host = 50
    t0 = time.perf_counter()
    for _ in range(n_host):
        runner.begin_batch(stream)
    plan_host_us = (time.perf_counter() - t0) / n_host * 1e6
    torch.cuda.synchronize()
    g_us, s_us = g_ms * 1e3, s_ms * 1e3
    # the dominant kernel is the one-launch layer (gpb_compose_layer): one
    # launch moves the layer's algorithmic bytes
    achieved = layer_bytes / (layer_ms * 1e-3) / 1e9
    out["us_per_layer"] = round(layer_ms * 1e3, 2)
    # the same figure from the headline region: (step - plan and clear) / L
    out["us_per_layer_from_step"] = round((ms_per_step - p_ms) * 1e3 / L, 2)
    out["pct_of_peak"] = round(100.0 * achieved / HBM_PEAK_GBS, 2)
    out["kernels_us"] = {"compose_layer": round(layer_ms * 1e3, 2),
                         "compose_gather": round(g_us, 2),
                         "current_row_scatter": round(s_us, 2),
                         "plan_build_with_staging_clear": round(p_ms * 1e3, 2),
                         "plan_build": round(p0_ms * 1e3, 2)}
    out["two_launch_layer"] = {
        "us_per_layer": round(two_ms * 1e3, 2),
        "pct_of_peak": round(100.0 * layer_bytes / (two_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "gather_pct_of_peak": round(100.0 * runner.gather_bytes() / (g_us * 1e-6) / 1e9
                                    / HBM_PEAK_GBS, 2)}
    out["plan_build_host_us"] = round(plan_host_us, 1)
    out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1),
                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(achieved / HBM_PEAK_GBS, 4),
                       "traffic": _traffic(a.workload),
                       "kernel": "compose_layer", "bytes_per_launch": layer_bytes}
    if a.no_extras:
        a.twin_index_bytes = 0
    else:
        _extras(a, out, runner, batch, stream, reps, L, s_ms, g_ms, lead)
        out["ceilings"] = _ceilings(gpb, stream, lead, achieved, batch, layer_bytes)
    assert int(runner.status.item()) == 0
    if a.calibration_copy_mib:
        n = a.calibration_copy_mib << 20
        x = torch.ones(n, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
    if a.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(batch, pools, curs, a.cpu_seconds)
    print(json.dumps(out), flush=True)


MIN_REGION_LAYERS = 200
MAX_REGION_REPS = 20      # repetitions of a many-layer loop per extra region
MEDIAN_STEPS = 10         # steps timed one by one for the median

# arenas cycled by the MALL-cold figure of one-layer workloads: 8 pools of
# 1.2 GB, far beyond the 256 MB MALL
COLD_ROTATIONS = 8


def _ceilings(gpb, stream, lead, achieved_gbs, batch, layer_bytes):
    """What plain streams reach on this GPU, as context for the roofline
    fraction: a write-only fill (the library's staging clear) and a torch
    device copy (read + write), each over 1 GiB buffers, four times what the
    256 MB MALL holds, in GPU-only regions; and a copy of the layer's own
    size -- the gather over contiguous pages of the workload's page size,
    reading and writing layer_bytes / 2 bytes each per launch -- cycled over
    enough buffer pairs that the MALL holds none of them, since a launch of
    tens of MB pays its ramp and tail on fewer bytes than a 1 GiB stream."""
    import torch
    n, reps = 1 << 30, 10
    x = torch.ones(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    fill_ms = _timed(stream, lambda: gpb.staging_clear(y, stream=stream), reps,
                     lead=lead(reps))
    copy_ms = _timed(stream, lambda: y.copy_(x), reps, lead=lead(reps))
    del x, y
    same = _layer_size_copy(gpb, stream, lead, batch.page_size, batch.row_bytes, layer_bytes)
    torch.cuda.empty_cache()
    fill_gbs = n / (fill_ms * 1e-3) / 1e9
    return {"buffer_bytes": n,
            "fill_write_gbs": round(fill_gbs, 1),
            "torch_copy_read_write_gbs": round(2 * n / (copy_ms * 1e-3) / 1e9, 1),
            "compose_layer_over_fill": round(achieved_gbs / fill_gbs, 4),
            "layer_size_copy": same,
            "compose_layer_over_layer_size_copy": round(achieved_gbs / same["read_write_gbs"],
                                                        4)}


def _layer_size_copy(gpb, stream, lead, page_rows, row_bytes, layer_bytes):
    """The library's gather over contiguous pages of page_rows x row_bytes,
    reading and writing layer_bytes / 2 bytes each per launch, cycled over
    enough buffer pairs (2 GiB of sources at least) that the MALL holds none
    of them: what a launch of the layer's size reaches, ramp and tail
    included."""
    import torch
    page = page_rows * row_bytes
    pages = max(1, layer_bytes // 2 // page)
    k = max(1, min(64, (2 << 30) // (pages * page)))
    srcs = [torch.ones(pages * page, dtype=torch.uint8, device="cuda") for _ in range(k)]
    dsts = [torch.empty_like(t) for t in srcs]
    tables = [gpb.Sources([(t, pages)]) for t in srcs]
    owner = torch.zeros(pages, dtype=torch.int32, device="cuda")
    src = torch.arange(pages, dtype=torch.int32, device="cuda")
    calls = k * max(1, -(-40 // k))

    def copies():
        for i in range(calls):
            gpb.compose_gather(dsts[i % k], tables[i % k], owner, src, pages, page_rows,
                               row_bytes, stream=stream)

    ms = _timed(stream, copies, 1, lead=lead(calls)) / calls
    del srcs, dsts, tables
    return {"bytes_per_launch": 2 * pages * page, "buffer_pairs": k, "us": round(ms * 1e3, 2),
            "read_write_gbs": round(2 * pages * page / (ms * 1e-3) / 1e9, 1)}


def _extras(a, out, runner, batch, stream, reps, L, s_ms, g_ms, lead):
    """Extra figures: the step replayed as one HIP graph; the layer in one
    launch; the layer-ahead prefetch split (the prefix gather can run a layer
    ahead, so the per-layer critical path is the consume: the fill or
    scatter plus the gather of the current pages), its halves alone and the
    whole batch run with the prefetch on a second stream; the fused fill; the
    scatter split over the writers; the index-key twin on the same plan."""
    import torch
    import gather_plan_build_amd as gpb
    import workloads

    def region(fn, calls_per_rep):
        return _timed(stream, fn, reps, lead=lead(reps * calls_per_rep))

    pre_ms = region(lambda: [runner.gather_prefix(l, stream) for l in range(L)], L) / L
    cur_ms = region(lambda: [runner.gather_current(l, stream) for l in range(L)], L) / L
    cons_ms = region(lambda: [runner.consume_fused(l, stream) for l in range(L)], L) / L
    fill_ms = region(lambda: [runner.fill(l, stream) for l in range(L)], L) / L
    layer_fill_ms = region(lambda: [runner.layer_fill(l, stream) for l in range(L)], L) / L
    own = runner.writer_rows_of(0)
    W = len(runner.writer_counts)
    wsc_ms = region(lambda: [runner.scatter_writers(l, own, stream) for l in range(L)],
                    W * L) / L
    del own
    # the whole batch with the layer-ahead prefetch on a second stream
    side = torch.cuda.Stream()
    pipe = {}
    for consume in ("fused", "scatter"):
        ms = region(lambda: runner.run_pipelined(L, stream, side, consume=consume),
                    4 * L + 2)
        pipe[consume] = ms
    # the same schedule on one stream, one launch per layer; and with the
    # fused fill in every consume
    ahead_ms = region(lambda: runner.run_layer_ahead(L, stream), L + 2)
    ahead_fill_ms = region(lambda: runner.run_layer_ahead(L, stream, fill=True), L + 2)
    cons_fill_ms = region(lambda: [runner.consume_fill(l, stream) for l in range(L)], L) / L
    serial_ms = region(lambda: runner.run(L, stream), L + 1)
    # the whole step captured once as a HIP graph and replayed: same kernels,
    # no per-launch host work
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        runner.run(L, side)
    torch.cuda.synchronize()
    graph.replay()
    graph_ms = region(graph.replay, 1)
    out["graph_replay"] = {"ms_per_step": round(graph_ms, 4),
                           "us_per_layer_incl_plan": round(graph_ms * 1e3 / L, 2)}
    del graph
    out["prefetch_split"] = {
        "prefix_gather_us": round(pre_ms * 1e3, 2),
        "current_gather_us": round(cur_ms * 1e3, 2),
        "split_over_one_shot": round((pre_ms + cur_ms) / g_ms, 4),
        "fused_fill_us": round(fill_ms * 1e3, 2),
        "consume_us": round((s_ms + cur_ms) * 1e3, 2),
        "consume_fused_us": round(cons_ms * 1e3, 2),
        "consume_with_fused_fill_us": round((fill_ms + cur_ms) * 1e3, 2),
        "one_launch_layer_with_fused_fill_us": round(layer_fill_ms * 1e3, 2),
        "fused_fill_bytes": 3 * batch.n_cur_tokens * batch.row_bytes
                            + 8 * batch.n_cur_tokens,
        "pipelined_ms_per_step": round(pipe["fused"], 4),
        "pipelined_us_per_layer_incl_plan": round(pipe["fused"] * 1e3 / L, 2),
        "pipelined_scatter_consume_ms_per_step": round(pipe["scatter"], 4),
        "layer_ahead_one_launch_ms_per_step": round(ahead_ms, 4),
        "layer_ahead_with_fused_fill_ms_per_step": round(ahead_fill_ms, 4),
        "consume_fused_with_fill_us": round(cons_fill_ms * 1e3, 2),
        "serial_one_launch_ms_per_step": round(serial_ms, 4)}
    out["writer_scatters"] = {"writers": W, "us_per_layer": round(wsc_ms * 1e3, 2),
                              "single_scatter_us": round(s_ms * 1e3, 2)}
    if batch.n_rotations == 1:
        # a workload that repeats one layer over the same arenas reads pool
        # pages the 256 MB MALL already holds: the same layer again over
        # COLD_ROTATIONS distinct pool and current-row arenas, cycled
        cpools, ccurs = workloads.make_values(batch, device="cuda",
                                              rotations=COLD_ROTATIONS, seed=batch.seed + 2)
        cold = gpb.ComposeRunner(gpb.BatchMeta.of(batch), cpools, ccurs, plan=runner.plan)
        cold.begin_batch(stream)
        R = COLD_ROTATIONS
        cold_ms = region(lambda: [cold.layer(l, stream) for l in range(R)], R) / R
        cold_b = cold.algorithmic_bytes_per_layer()
        out["mall_cold"] = {"rotations": R, "us_per_layer": round(cold_ms * 1e3, 2),
                            "pct_of_peak": round(100.0 * cold_b / (cold_ms * 1e-3) / 1e9
                                                 / HBM_PEAK_GBS, 2)}
        assert int(cold.status.item()) == 0
        del cold, cpools, ccurs
    if a.twin_index_bytes:
        rb = a.twin_index_bytes
        ipools, icurs = workloads.make_values(batch, device="cuda", row_bytes=rb,
                                              value_kind="bytes", seed=batch.seed + 1)
        twin = gpb.ComposeRunner(
            gpb.BatchMeta(batch.bs, batch.page_size, rb, batch.n_pool_pages,
                          batch.n_pool_entries, batch.n_writers, batch.staging_cap_pages,
                          batch.prefix_pages, batch.cur_tokens, batch.req_pages),
            ipools, icurs, plan=runner.plan)
        twin.begin_batch(stream)
        t_ms = region(lambda: [twin.layer(l, stream) for l in range(L)], L) / L
        t2_ms = region(lambda: [twin.layer_two_launch(l, stream) for l in range(L)],
                       2 * L) / L
        tb = twin.algorithmic_bytes_per_layer()
        sep_ms = region(lambda: [(runner.layer(l, stream), twin.layer(l, stream))
                                 for l in range(L)], 2 * L) / L
        both_ms = region(lambda: [gpb.layer_groups([runner, twin], l, stream)
                                  for l in range(L)], L) / L
        both2_ms = region(lambda: [gpb.layer_groups_two_launch([runner, twin], l, stream)
                                   for l in range(L)], 2 * L) / L
        both_b = runner.algorithmic_bytes_per_layer() + tb
        out["index_twin"] = {"row_bytes": rb, "us_per_layer": round(t_ms * 1e3, 2),
                             "algorithmic_bytes_per_layer": tb,
                             "gbs": round(tb / (t_ms * 1e-3) / 1e9, 1),
                             "pct_of_peak": round(100.0 * tb / (t_ms * 1e-3) / 1e9
                                                  / HBM_PEAK_GBS, 2),
                             "two_launch_us_per_layer": round(t2_ms * 1e3, 2),
                             "token_and_twin_separate_us": round(sep_ms * 1e3, 2),
                             "token_and_twin_grouped_us": round(both_ms * 1e3, 2),
                             "grouped_gbs": round(both_b / (both_ms * 1e-3) / 1e9, 1),
                             "grouped_pct_of_peak": round(100.0 * both_b / (both_ms * 1e-3)
                                                          / 1e9 / HBM_PEAK_GBS, 2),
                             "token_and_twin_grouped_two_launch_us": round(both2_ms * 1e3,
                                                                           2)}
        assert int(twin.status.item()) == 0
        del ipools, icurs
        twin_copy = _layer_size_copy(gpb, stream, lead, batch.page_size, rb, tb)
        out["index_twin"]["layer_size_copy"] = twin_copy
        out["index_twin"]["over_layer_size_copy"] = round(
            tb / (t_ms * 1e-3) / 1e9 / twin_copy["read_write_gbs"], 4)
        del twin
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
