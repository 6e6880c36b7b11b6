"""Build libmqconv.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Each .hip translation unit is compiled to an object in parallel, then all are
linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmqconv.so")
SOURCES = ["quantize.hip", "layout.hip", "gemm_fwd.hip", "gemm_fwd_mx.hip", "gemm_dgrad.hip", "gemm_dgrad_mx.hip", "gemm_dgrad_mx_relaid.hip", "gemm_wgrad.hip", "gemm_wgrad_sub.hip", "gemm_plain.hip",
           "naive.hip", "cuyckens.hip", "nvfp.hip", "mqconv_api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off (see the design notes on numerics)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-unused-value",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _includes(path: str, seen: set) -> set:
    """Local headers a source includes, transitively (#include "...")."""
    import re
    for name in re.findall(r'^#include "([^"]+)"', open(path).read(), flags=re.M):
        for d in (CSRC, os.path.join(ROOT, "include")):
            h = os.path.join(d, name)
            if os.path.exists(h) and h not in seen:
                seen.add(h)
                _includes(h, seen)
    return seen


def _stale(src: str, obj: str) -> bool:
    """An object is stale when older than its source or a header it includes."""
    if not os.path.exists(obj):
        return True
    path = os.path.join(CSRC, src)
    deps = [path, *_includes(path, set())]
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if incremental and not _stale(src, obj):
        return obj
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every translation unit (incremental: only those whose object is
    older than its source or a header) and link libmqconv.so."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, incremental), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)
