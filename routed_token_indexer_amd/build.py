"""Build the HIP library ``libmisa.so`` in-tree for gfx950.

Usage: ``python -m routed_token_indexer_amd.build`` (or ``build()`` from Python).
hipcc cross-compiles the device code without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmisa.so")
SOURCES = ["abi.hip", "pool.hip", "route.hip", "score.hip", "topk.hip", "topk_split.hip", "block.hip", "pivot.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    # device code linked and optimized as a whole at link time: the selection
    # kernels come out with fewer registers (no spills at 64 per lane)
    "-fgpu-rdc",
    # no packed-fp32 VALU instructions on the device (hipcc's host pass does not
    # know the feature and says so; that message is harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source to an object in parallel, then link ``libmisa.so``."""
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs = []
    objs = []
    t0 = time.time()
    for src in SOURCES:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [hipcc()] + [f for f in FLAGS if f != "-shared"] + inc + ["-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        while sum(p.poll() is None for _, p in procs) >= jobs:
            time.sleep(0.05)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-fgpu-rdc", "--hip-link", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
