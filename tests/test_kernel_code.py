"""Checks of the built gfx950 code itself (CPU only: llvm-objdump and
llvm-readelf over every gfx950 code object in libmqconv.so).

1. The 2 x 16 FP6 conversion instruction writes its six result registers
   while it still reads its two 16-register operands, so a result register
   that shares a register with an operand corrupts codes (an in-bounds check
   of the instruction's lane layout showed exactly that when the compiler
   placed the result inside the first operand). mx_common.h keeps the
   operands live across the instruction; no conversion may overlap.
2. No kernel uses scratch memory: a kernel whose registers spill to scratch
   runs several times slower (the backward-data GEMM with the MX epilogue did
   on its 256 x 128 tile), and the GEMM kernels keep their register budget of
   two waves per SIMD."""
import os
import re
import struct
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest
import yaml

import microscaling_quantized_convolution_mxq_amd as mq

BIN = "/opt/rocm/llvm/bin"
CVT = re.compile(r"v_cvt_scalef32_2xpk16_b?f6_f32 v\[(\d+):(\d+)\], v\[(\d+):(\d+)\], v\[(\d+):(\d+)\]")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

pytestmark = pytest.mark.skipif(not os.path.exists(os.path.join(BIN, "llvm-objdump")),
                                reason="LLVM tools of the ROCm toolchain not installed")


def gfx950_code_objects(path):
    """The gfx950 entries of every clang offload bundle in the file."""
    data = open(path, "rb").read()
    i = data.find(MAGIC)
    while i >= 0:
        n = struct.unpack_from("<Q", data, i + len(MAGIC))[0]
        off = i + len(MAGIC) + 8
        for _ in range(n):
            o, size, tlen = struct.unpack_from("<QQQ", data, off)
            off += 24
            triple = data[off:off + tlen].decode()
            off += tlen
            if triple.endswith("gfx950") and size:
                yield data[i + o:i + o + size]
        i = data.find(MAGIC, i + len(MAGIC))


def run_tool(tool, args, code_object: bytes) -> str:
    with tempfile.NamedTemporaryFile(suffix=".co") as f:
        f.write(code_object)
        f.flush()
        return subprocess.run([os.path.join(BIN, tool), *args, f.name], capture_output=True, text=True,
                              check=True).stdout


def over_library(fn):
    if not os.path.exists(mq.LIB_PATH):
        pytest.skip("libmqconv.so is not built")
    objs = list(gfx950_code_objects(mq.LIB_PATH))
    assert objs, "no gfx950 code object found in the library"
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return [r for rs in ex.map(fn, objs) for r in rs]


def fp6_conversions(code_object: bytes):
    text = run_tool("llvm-objdump", ["-d", "--mcpu=gfx950"], code_object)
    return [tuple(map(int, m.groups())) + (m.group(0),) for m in CVT.finditer(text)]


def kernel_metadata(code_object: bytes):
    text = run_tool("llvm-readelf", ["--notes"], code_object)
    start = text.index("---", text.index("AMDGPU Metadata"))
    end = text.index("\n...", start)
    return yaml.safe_load(text[start:end])["amdhsa.kernels"]


def test_fp6_conversion_results_never_overlap_operands():
    found = over_library(fp6_conversions)
    # the FP6 element formats are built (quantizer, MX epilogues, comparators)
    assert len(found) > 100
    bad = [text for d0, d1, a0, a1, b0, b1, text in found
           if not (d1 < a0 or d0 > a1) or not (d1 < b0 or d0 > b1)]
    assert not bad, f"{len(bad)} FP6 conversions whose result overlaps an operand, e.g. {bad[:3]}"


def test_no_kernel_spills_to_scratch():
    kernels = over_library(kernel_metadata)
    assert len(kernels) > 1000
    spills = [k[".name"] for k in kernels
              if k.get(".private_segment_fixed_size", 0) or k.get(".vgpr_spill_count", 0)]
    assert not spills, f"{len(spills)} kernels use scratch memory, e.g. {spills[:3]}"
    gemm = [k for k in kernels if "mx_gemm_kernel" in k[".name"]]
    assert gemm
    wide = [(k[".name"], k[".vgpr_count"], k.get(".agpr_count", 0)) for k in gemm
            if k[".vgpr_count"] + k.get(".agpr_count", 0) > 256]
    assert not wide, f"{len(wide)} GEMM kernels exceed 256 registers per lane, e.g. {wide[:3]}"
