"""Build libmolora.so (gfx950) in-tree with hipcc.

    python -m token_adapter_routing_amd.build        # or __graft_entry__.build()

Each source compiles to an object under _build/ in parallel, then hipcc links the shared
library next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmolora.so")
SOURCES = ["capi.cpp", "plan.cpp", "route.hip", "dispatch.hip", "apply.hip", "dense.hip", "gsplit.hip", "backward.hip", "xf.hip", "xfmr.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is expected
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    return p.returncode, out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmds.append([HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose and out.strip():
            print(out)
        if rc != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs, "-L/opt/rocm/lib", "-lrocblas",
                    "-Wl,-rpath,/opt/rocm/lib"])
    if rc != 0:
        raise RuntimeError(f"link failed\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
