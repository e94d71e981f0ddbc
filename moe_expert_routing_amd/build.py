"""Build libmoe_route.so (gfx950) in-tree with hipcc.

    python -m moe_expert_routing_amd.build

Every call compiles all sources again.  The library lands next to this file,
so it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_route.so")
SOURCES = ["route_api.cpp", "route_generic.hip", "route_fast.hip", "route_row.hip", "fused_router.hip",
           "fused_router_small.hip", "route_dispatch.hip", "route_post.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source (in parallel, one hipcc per source) and link."""
    jobs = jobs or max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with tempfile.TemporaryDirectory(prefix="moe_route_build_") as tmp:
        cmds, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmds.append([HIPCC, *CFLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        if verbose:
            for cmd in cmds:
                print(" ".join(cmd), flush=True)
        with ThreadPoolExecutor(jobs) as ex:
            for rc, cmd in zip(ex.map(subprocess.call, cmds), cmds):
                if rc != 0:
                    raise subprocess.CalledProcessError(rc, cmd)
        out_tmp = os.path.join(tmp, "libmoe_route.so")
        cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", out_tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
