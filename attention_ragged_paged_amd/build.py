"""Build librpa.so (gfx950 only) in-tree with hipcc.

Every .hip source under csrc/ is compiled to an object in parallel, then linked into
attention_ragged_paged_amd/librpa.so.  Run ``python -m attention_ragged_paged_amd.build``
or call ``build()``.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librpa.so")
OBJ_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU forms are kept out of the device code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    procs = []
    objs = []
    for src in sources:
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the device-only target feature; that note is noise
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l or "error" in l]
        if lines and (verbose or p.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
