"""Host-sanitizer build of libmqconv.so, for the CPU tests of the host-side
validation and launch-set-up code.

The translation units that hold the C ABI's argument validation and the
launch set-up of the quantizer, the im2col and the comparison paths are
compiled again with AddressSanitizer and UndefinedBehaviorSanitizer on their
host code only (device code is built as usual), then linked with the regular
objects of the GEMM units into _build/sanitize/libmqconv_sanitize.so. A test
loads that library (MQCONV_LIB) in a Python process that preloads the
sanitizer runtime and runs the validation tests; any report fails them.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

from microscaling_quantized_convolution_mxq_amd import build as b

SANITIZED = ["mqconv_api.hip", "quantize.hip", "layout.hip", "naive.hip", "nvfp.hip"]
OUT = os.path.join(b.BUILD, "sanitize")
LIB = os.path.join(OUT, "libmqconv_sanitize.so")
# host-only sanitizer flags: each one after -Xarch_host
HOST_SAN = []
for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer"):
    HOST_SAN += ["-Xarch_host", flag]


def runtime() -> str:
    """The clang AddressSanitizer runtime of the ROCm toolchain ('' if absent)."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else ""


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    if not b._stale(src, obj):
        return obj
    cmd = [b.HIPCC, *b.FLAGS, *HOST_SAN, "-c", os.path.join(b.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Build the sanitized library (the regular objects must be built)."""
    os.makedirs(OUT, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(len(SANITIZED)) as ex:
        objs = list(ex.map(_compile, SANITIZED))
    for src in b.SOURCES:
        if src not in SANITIZED:
            obj = os.path.join(b.BUILD, os.path.splitext(src)[0] + ".o")
            if b._stale(src, obj):
                raise RuntimeError(f"{obj} is missing or stale: build the library first")
            objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [b.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, "-shared-libsan", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
