"""Compile libw4a16.so in-tree with hipcc for gfx950 (no JIT, no cache outside the tree)."""
from __future__ import annotations

import concurrent.futures as _cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_NAME = "libw4a16.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
# (source, extra defines): the codec kernels are one source compiled once per codec
UNITS = [
    ("csrc/w4a16_gemv.hip", []),
    ("csrc/w4a16_chain.hip", []),
    ("csrc/w4a16_codec_kernels.hip", ["-DW4A16_CODEC_ID=1"]),
    ("csrc/w4a16_codec_kernels.hip", ["-DW4A16_CODEC_ID=2"]),
    ("csrc/w4a16_codec_kernels.hip", ["-DW4A16_CODEC_ID=3"]),
    ("csrc/w4a16_codec_kernels.hip", ["-DW4A16_CODEC_ID=4"]),
    ("csrc/w4a16_codec.cpp", []),
    ("csrc/w4a16_kv.hip", []),
    ("csrc/w4a16_pack.cpp", []),
]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 VALU forms anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 16 dwords of explicit kernel arguments arrive in scalar
    # registers when a wave starts, instead of by scalar loads from the
    # argument segment (a memory round trip before the first weight load)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the W4A16 library needs ROCm's hipcc to build")


def _jobs() -> int:
    for var in ("MAX_JOBS", "CMAKE_BUILD_PARALLEL_LEVEL"):
        v = os.environ.get(var, "")
        if v.isdigit() and int(v) > 0:
            return min(int(v), 16)
    return max(1, min(len(UNITS), len(os.sched_getaffinity(0))))


def build(verbose: bool = False) -> str:
    """Always recompile every unit (in parallel), link, and write the library
    atomically next to this file."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="w4a16_build_") as objdir:
        def compile_unit(i_unit):
            i, (src, defs) = i_unit
            obj = os.path.join(objdir, "u%d.o" % i)
            cmd = [hipcc(), *HIP_FLAGS, "-c", *defs, *inc, os.path.join(PKG_DIR, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed on %s %s" % (src, " ".join(defs)))
            return obj

        with _cf.ThreadPoolExecutor(max_workers=_jobs()) as ex:
            objs = list(ex.map(compile_unit, enumerate(UNITS)))
        cmd = [hipcc(), *HIP_FLAGS, "-shared", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed linking %s" % LIB_NAME)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
