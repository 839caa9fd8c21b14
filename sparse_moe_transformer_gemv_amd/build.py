"""Build libflint_moe.so in-tree with hipcc for gfx950 only.

    python -m sparse_moe_transformer_gemv_amd.build

The library is the product: every kernel of the MoE layer is in csrc/*.hip,
and the C ABI (include/flint_moe.h) is implemented in csrc/flint_moe.cpp.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libflint_moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                "-I", INCLUDE, "-I", CSRC]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "flint_moe.cpp")]


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source (in parallel) and link libflint_moe.so."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        if src.endswith(".hip"):
            cmd = [HIPCC, *DEVICE_FLAGS, *COMMON_FLAGS, "-c", src, "-o", obj]
        else:
            cmd = [HIPCC, *COMMON_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(f) for f in failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *DEVICE_FLAGS, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
