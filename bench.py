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
layers, over the measured step time).  Per-kernel durations come from HIP
events recorded around every launch on the launch stream, inside the timed
region.  ``cpu_baseline`` times the CPU oracle on a bounded sample of the
same layers on this host.
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
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="traced",
                    choices=["traced", "opaque", "medium", "multi_source", "tiny"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the CPU oracle sample (0 disables it)")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time whole steps only (no per-launch events)")
    return ap.parse_args()


def _source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gather_plan_build_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _traffic(workload, gather_launch_bytes):
    """HBM bytes per gather launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "compose_gather_%s_counters.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != _source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(batch, pools, curs, budget_s):
    """The CPU oracle (plain C loops, one thread) on the same batch: the plan
    once, then layers until the budget is spent.  Returns the JSON object."""
    import numpy as np
    import oracle
    orc = oracle.default()
    t0 = time.perf_counter()
    want = oracle.plan_for(batch, orc)
    plan_s = time.perf_counter() - t0
    staging = np.empty(batch.staging_rows_total * batch.row_bytes, np.uint8)
    host_pools, host_curs = {}, {}
    per_layer = []
    spent = 0.0
    layer = 0
    while layer < batch.n_layers and (spent < budget_s or layer == 0):
        k = layer % len(pools)
        if k not in host_pools:
            host_pools[k] = pools[k].cpu().numpy().reshape(-1)
            host_curs[k] = curs[k].cpu().numpy()
        t0 = time.perf_counter()
        oracle.layer_for(batch, want, host_pools[k], host_curs[k], staging, orc)
        dt = time.perf_counter() - t0
        per_layer.append(dt)
        spent += dt
        layer += 1
    S, T = batch.n_req_pages, batch.n_cur_tokens
    PS, RB = batch.page_size, batch.row_bytes
    layer_bytes = (2 * S * PS * RB + 2 * T * RB + 8 * S + 4 * T
                   + 8 * (batch.n_pool_entries + batch.n_writers))
    med = sorted(per_layer)[len(per_layer) // 2]
    return {"value": round(layer_bytes / med / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "us_per_layer": round(med * 1e6, 1),
            "plan_us": round(plan_s * 1e6, 1),
            "sample": "%d of %d layers of the %s workload (median per layer; plan "
                      "once), single-threaded C oracle: zero staging, scatter "
                      "current rows, gather every page" % (len(per_layer),
                                                           batch.n_layers, batch.name),
            "cpu_model": _cpu_model(), "host_threads_available": os.cpu_count()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    a = _args()
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

    def step(ev):
        if ev is None:
            runner.run(L, stream)
            return
        ev["plan"][0].record(stream)
        runner.begin_batch(stream)
        ev["plan"][1].record(stream)
        marks = ev["marks"]
        for layer in range(L):
            runner.scatter(layer, stream)
            marks[2 * layer].record(stream)
            runner.gather(layer, stream)
            marks[2 * layer + 1].record(stream)

    def new_events():
        E = torch.cuda.Event
        return {"plan": [E(enable_timing=True), E(enable_timing=True)],
                "marks": [E(enable_timing=True) for _ in range(2 * L)]}

    for _ in range(a.warmup):
        step(None)
    torch.cuda.synchronize()

    evs = [None if a.no_kernel_events else new_events() for _ in range(a.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(a.steps):
        step(evs[s])
    stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / a.steps
    assert int(runner.status.item()) == 0, "a kernel flagged a bad descriptor or row"

    layer_bytes = runner.algorithmic_bytes_per_layer()
    value_gbs = layer_bytes * L / (ms_per_step * 1e-3) / 1e9
    out = {"metric": METRIC, "value": round(value_gbs, 1), "unit": "GB/s",
           "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
           "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
           "config": {"workload": "%s: bs=%d, %d current tokens, %d dense slots, "
                                  "%d-token pages, %d-byte rows, %d layers, plan once "
                                  "per batch" % (batch.name, batch.bs, batch.n_cur_tokens,
                                                 batch.n_req_pages, batch.page_size,
                                                 batch.row_bytes, L),
                      "global_batch": batch.bs, "seq_len": None,
                      "parallelism": "single GPU",
                      "algorithmic_bytes_per_layer": layer_bytes}}
    if not a.no_kernel_events:
        gather_ms, scatter_ms, plan_ms = [], [], []
        for ev in evs:
            m = ev["marks"]
            plan_ms.append(ev["plan"][0].elapsed_time(ev["plan"][1]))
            scatter_ms.append(ev["plan"][1].elapsed_time(m[0]))
            for layer in range(L):
                if layer:
                    scatter_ms.append(m[2 * layer - 1].elapsed_time(m[2 * layer]))
                gather_ms.append(m[2 * layer].elapsed_time(m[2 * layer + 1]))
        g_us = 1e3 * sum(gather_ms) / len(gather_ms)
        s_us = 1e3 * sum(scatter_ms) / len(scatter_ms)
        compose_us = g_us + s_us
        g_bytes = runner.gather_bytes()
        achieved = g_bytes / (g_us * 1e-6) / 1e9
        traffic = _traffic(a.workload, g_bytes)
        out["us_per_layer"] = round(compose_us, 2)
        out["compose_gbs"] = round(layer_bytes / (compose_us * 1e-6) / 1e9, 1)
        out["pct_of_peak"] = round(100.0 * out["compose_gbs"] / HBM_PEAK_GBS, 2)
        out["kernels_us"] = {"compose_gather": round(g_us, 2),
                             "current_row_scatter": round(s_us, 2),
                             "plan_build_and_staging_clear": round(
                                 1e3 * sum(plan_ms) / len(plan_ms), 2)}
        out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": traffic,
                           "kernel": "compose_gather", "bytes_per_launch": g_bytes}
    if a.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(batch, pools, curs, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
