"""Build libgpb.so in-tree with hipcc for gfx950.

    python gather_plan_build_amd/build.py [--define NAME=VALUE ...] [--out PATH]

(run as a script: importing the package needs the library this builds)

Every HIP source under csrc/ goes into one shared library next to this file.
Packed-FP32 instructions are switched off for all device code.
"""
import argparse
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgpb.so")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def command(out, defines=()):
    # code object v5: loadable by the HIP runtime torch bundles as well as by
    # the system ROCm one; the library binds to whichever the process loaded.
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-mcode-object-version=5", "-O3",
           "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Werror",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # the leading kernel arguments arrive in scalar registers at wave
           # launch instead of being read from the argument segment
           "-mllvm", "-amdgpu-kernarg-preload-count=16",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    cmd += ["-D" + d for d in defines]
    return cmd + ["-o", out] + sources()


def build(out=LIB, defines=()):
    """Compile every source; replaces ``out`` atomically."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(command(tmp, defines), check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--define", "-D", action="append", default=[])
    ap.add_argument("--out", default=LIB)
    a = ap.parse_args()
    print(build(a.out, a.define))
