"""Compile the HIP library ``libmoe.so`` in-tree for gfx950 with hipcc.

Every source compiles to its own object in parallel, then one link."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["route.hip", "permute.hip", "route_plan.hip", "ffn.hip", "ffn_lowbit.hip", "ffn_mx.hip", "combine.hip",
           "noalloc.hip", "abi.cpp"]
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
         # keep the compiler from emitting packed-fp32 VALU instructions
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in l and l.strip()]
    return r.returncode, msgs


def build(verbose: bool = False) -> str:
    """Build libmoe.so from every source (always recompiles)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        cmds = [[hipcc, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for cmd, (rc, msgs) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                sys.stderr.write("\n".join(msgs) + "\n")
                raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-3]}")
            if verbose and msgs:
                print("\n".join(msgs))
        out = LIB + ".tmp"
        rc, msgs = _run([hipcc, *FLAGS, "-shared", *objs, "-o", out])
        if rc != 0:
            sys.stderr.write("\n".join(msgs) + "\n")
            raise RuntimeError(f"hipcc link failed ({rc})")
    os.replace(out, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
