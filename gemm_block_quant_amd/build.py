"""Build libquantgemm.so (HIP, gfx950) in the package directory.

    python -m gemm_block_quant_amd.build [-v] [--incremental] [--sanitize]

Every call compiles from source (hipcc cross-compiles without a GPU).  With
--incremental, objects newer than their source and every header are kept.
--sanitize builds a copy whose host code is instrumented for AddressSanitizer
and UndefinedBehaviorSanitizer (gemm_block_quant_amd/_asan/libquantgemm.so, for
host-only tests; the device code is unchanged).
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


# Host-side sanitizers (each -fsanitize= placed after -Xarch_host: device code is not instrumented).
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_DIR = os.path.join(HERE, "_asan")


def build(verbose: bool = False, jobs: int = 8, incremental: bool = False, sanitize: bool = False) -> str:
    objs = []
    procs = []
    bdir = ASAN_DIR if sanitize else os.path.join(HERE, "_build")
    lib = os.path.join(ASAN_DIR, "libquantgemm.so") if sanitize else LIB
    os.makedirs(bdir, exist_ok=True)
    newest_header = max((os.path.getmtime(h) for h in _headers()), default=0.0)
    for src in sources():
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        objs.append(obj)
        if incremental and os.path.exists(obj) and \
                os.path.getmtime(obj) > max(os.path.getmtime(src), newest_header):
            continue
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-Wno-unused-function", "-c", src, "-o", obj] + DEVICE_FLAGS + (SANITIZE_FLAGS if sanitize else [])
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _drain(procs)
    _drain(procs)
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + \
        (["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"] if sanitize else [])
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


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
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv, sanitize="--sanitize" in sys.argv))
