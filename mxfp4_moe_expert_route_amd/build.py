"""Build libmxfp4moe.so (HIP, gfx950) in-tree with hipcc.

Each .hip source under csrc/ is compiled to an object in _build/ (in
parallel), then linked into mxfp4_moe_expert_route_amd/libmxfp4moe.so.  The
library is written to a temporary name and renamed, so a process that has the
old one loaded is never handed a half-written file.
"""

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmxfp4moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


# per-source flags.  decode_layer.hip: no atomic aggregation across a wave
# (the kernel's atomics run on one lane, and the aggregated form reads each
# answer at once, which would put every queue claim's round trip on the path
# of the stage barriers)
FILE_FLAGS = {"decode_layer.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), r.stdout))
    if verbose and out.strip():
        print(out)


def build(verbose=False, jobs=None):
    """Compile every HIP source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _run([HIPCC] + FLAGS + FILE_FLAGS.get(os.path.basename(so[0]), [])
                                    + ["-c", so[0], "-o", so[1]], verbose),
                    zip(srcs, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
