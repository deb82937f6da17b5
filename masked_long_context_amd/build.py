"""Build libbdattn.so (gfx950) in-tree with hipcc.

    python -m masked_long_context_amd.build [--verbose] [--resource-usage]

Every source is compiled to an object in parallel, then linked into
masked_long_context_amd/libbdattn.so.  The library links the HIP runtime by
its soname, so inside a process that already loaded PyTorch's HIP runtime it
binds to that same runtime (and to torch's streams and device pointers).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libbdattn.so")
BUILD = os.path.join(PKG, "_build")

SOURCES = ["plan.cpp", "capi.cpp", "noalloc.hip", "kernels/fwd.hip", "kernels/bwd.hip", "kernels/aux.hip"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
          "-Wall", "-Wno-unused-function",
          # packed fp32 ALU forms stay off (host pass warns that it does not know the feature)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libbdattn.so)")


# Per-source scheduler choice: the attention kernels gain from LLVM's ILP-first
# machine scheduler (operand loads hoisted further ahead of their MFMAs).  Of
# the other strategies, max-memory-clause and iterative-ilp measured slower.
ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
EXTRA = {"kernels/bwd.hip": ILP, "kernels/fwd.hip": ILP}


def _compile(src: str, resource_usage: bool, verbose: bool) -> str:
    obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
    cmd = [hipcc()] + COMMON + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if resource_usage and src.endswith(".hip"):
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "is not a recognized feature")
    err = "\n".join(l for l in r.stderr.splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{err}")
    if verbose or resource_usage:
        if err.strip():
            print(f"--- {src}\n{err}", file=sys.stderr)
    return obj


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, resource_usage, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    args = ap.parse_args()
    print(build(args.verbose, args.resource_usage))
