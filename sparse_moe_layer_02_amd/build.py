"""Build the gfx950 HIP library ``libmoe_mi355x.so`` in-tree with hipcc.

Every ``csrc/*.hip`` file is compiled to an object for gfx950 (in parallel),
then linked into a shared library next to this file.  Packed fp32 arithmetic
is disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src, obj):
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device feature flag; that warning is expected
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (os.path.basename(src), err))
    return err


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        for s, msg in zip(srcs, ex.map(_compile, srcs, objs)):
            if msg.strip() and verbose:
                print("%s:\n%s" % (os.path.basename(s), msg))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
