"""Builds libml4dsa.so (the HIP kernels + C-ABI shim) in-tree for gfx950 with hipcc."""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libml4dsa.so")
SOURCES = ["abi.cpp", "indexer.hip", "topk.hip", "sparse_mla.hip", "cache_write.hip",
           "merge.hip", "static_ws.hip", "probe.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


# Per-source extras: the indexer's MFMA results feed VALU work directly, so they are kept
# in VGPRs rather than accumulation registers (no copy per element).
EXTRA = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        jobs.append((obj, [hipcc, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src),
                           "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[j[0] for j in jobs],
          "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
