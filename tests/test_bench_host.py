"""Host-side parts of bench.py on the CPU: the oracle baseline legs on the
tiny workload (with host tensors), the multi-GPU refusal, and the profile
summaries' command strings.  Nothing here touches a GPU."""
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cpu_baseline_legs_on_the_tiny_workload():
    b = workloads.make_batch("tiny")
    pools, curs = workloads.make_values(b, device="cpu")
    r = bench.cpu_baseline(b, pools, curs, 0.2, threads=2)
    for leg in (r, r["threaded"], r["concurrent_layers"]):
        assert leg["kind"] == "oracle" and leg["unit"] == "GB/s" and leg["value"] > 0
    assert r["cores"] == 1
    assert r["threaded"]["cores"] == 2 and r["concurrent_layers"]["cores"] == 2
    assert r["us_per_layer"] > 0 and r["threaded"]["us_per_layer"] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_profile_commands_name_the_workload_and_output_dir():
    c = bench._profile_commands(os.path.join(ROOT, "out", "prof_trace"), "opaque")
    assert "-d $REPO/out/prof_trace" in c["trace"]
    assert "bench.py --workload opaque" in c["trace"]
    assert c["summary"].endswith("--workload opaque")
    t = bench._profile_commands(os.path.join(ROOT, "out", "prof_trace"))
    assert "--workload" not in t["trace"]


def test_kernel_digest_reads_the_library_code_objects(tmp_path):
    """The counters' key: the digest of the gfx950 kernel code in libgpb.so
    (found through its offload bundles) is a stable 16-hex-digit value, not
    the digest of nothing, and the same for a byte copy of the library."""
    import hashlib
    import shutil
    d = bench._kernel_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    assert d != hashlib.sha256(b"").hexdigest()[:16]
    copy = tmp_path / "libcopy.so"
    shutil.copyfile(bench.LIB, copy)
    assert bench._kernel_digest(str(copy)) == d
    with open(bench.LIB, "rb") as f:
        data = f.read()
    assert bench._elf_section(data, ".hip_fatbin") is not None
    assert bench._elf_section(data, ".no_such_section") is None
