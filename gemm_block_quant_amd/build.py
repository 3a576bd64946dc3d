"""Build libquantgemm.so (HIP, gfx950) in the package directory.

    python -m gemm_block_quant_amd.build [-v] [--incremental]

Every call compiles from source (hipcc cross-compiles without a GPU).  With
--incremental, objects newer than their source and every header are kept.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libquantgemm.so")
ARCH = os.environ.get("QG_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU instructions are disabled for all device code; plain fp32
# arithmetic is used instead.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _headers():
    root = os.path.dirname(HERE)
    return glob.glob(os.path.join(HERE, "csrc", "*.h")) + glob.glob(os.path.join(root, "include", "*.h"))


def build(verbose: bool = False, jobs: int = 8, incremental: bool = False) -> str:
    objs = []
    procs = []
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    newest_header = max((os.path.getmtime(h) for h in _headers()), default=0.0)
    for src in sources():
        obj = os.path.join(HERE, "_build", os.path.basename(src) + ".o")
        objs.append(obj)
        if incremental and os.path.exists(obj) and \
                os.path.getmtime(obj) > max(os.path.getmtime(src), newest_header):
            continue
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-Wno-unused-function", "-c", src, "-o", obj] + DEVICE_FLAGS
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _drain(procs)
    _drain(procs)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def _drain(procs):
    failed = None
    while procs:
        src, p = procs.pop(0)
        out = p.communicate()[0].decode(errors="replace")
        lines = [l for l in out.splitlines() if "is not a recognized feature for this target" not in l]
        if lines:
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0 and failed is None:
            failed = src
    if failed:
        raise RuntimeError("hipcc failed on %s" % failed)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))
