"""Build libpagedkv.so (HIP kernels for gfx950 + host allocator) in-tree.

Usage: ``python -m paged_kv_cache_244_amd.build`` or ``build()`` from Python;
``--timeline`` (``build(timeline=True)``) builds the instrumented
libpagedkv_timeline.so instead.  Every call recompiles.  Only gfx950 code
objects are produced.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpagedkv.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
# The same sources with the decode kernels' per-wave timeline compiled in
# (-DPKV_WAVE_TIMELINE): a measurement tool, never loaded by the product path.
TIMELINE_LIB_PATH = os.path.join(PKG_DIR, "libpagedkv_timeline.so")

HIP_SOURCES = ["pa_decode.hip", "pa_decode_valu.hip", "pa_decode_mfma.hip", "pa_decode_fused.hip",
               "pa_decode_reduce.hip",
               "pa_prefill.hip", "kv_cache_ops.hip", "read_probe.hip", "check_tables.hip"]
HOST_SOURCES = ["allocator.cpp", "decode_plan.cpp", "errors.cpp"]

# Device code: gfx950 only; packed-fp32 instructions disabled (the compiler
# would otherwise form v_pk_* fp32 ops from scalar float code).
DEVICE_FLAGS = [
    "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source additions.  The prefill kernel's maxima run over scores that are
# never NaN (finite fp16 inputs, -inf for masked tokens): without NaN handling
# the compiler drops the quieting copy it otherwise puts before each max.
SOURCE_FLAGS = {"pa_prefill.hip": ["-fno-honor-nans"]}
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}",
                f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpagedkv.so)")


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(jobs: int = min(8, os.cpu_count() or 4), timeline: bool = False) -> str:
    """Compile every source to an object, then link the shared library
    (``timeline``: the instrumented libpagedkv_timeline.so instead)."""
    obj_dir = os.path.join(ROOT, "_build", "timeline") if timeline else os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    extra = ["-DPKV_WAVE_TIMELINE"] if timeline else []
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(obj_dir, src + ".o")
        cmds.append([cc, "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj] + DEVICE_FLAGS + COMMON_FLAGS
                    + SOURCE_FLAGS.get(src, []) + extra)
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(obj_dir, src + ".o")
        cmds.append([cc, "-c", "-x", "c++", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS)
        objs.append(obj)
    procs = []
    for cmd in cmds:
        print("+", " ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
        if len(procs) >= jobs:
            if procs.pop(0).wait() != 0:
                raise RuntimeError("compilation failed")
    for p in procs:
        if p.wait() != 0:
            raise RuntimeError("compilation failed")
    out = TIMELINE_LIB_PATH if timeline else LIB_PATH
    tmp = out + ".tmp"
    _run([cc, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs)
    os.replace(tmp, out)
    if not timeline:
        build_c_abi_test(cc)
    return out


C_ABI_TEST_SRC = os.path.join(ROOT, "tests", "c_abi_decode.cpp")
C_ABI_TEST_BIN = os.path.join(ROOT, "tests", "c_abi_decode")


def build_c_abi_test(cc: str) -> str:
    """The host program that drives the library through its C ABI alone (tests/):
    host C++ linked against libpagedkv.so and the HIP runtime, found next to it."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(cc)))
    tmp = C_ABI_TEST_BIN + ".tmp"
    _run([cc, "-x", "c++", C_ABI_TEST_SRC, "-o", tmp, "-O2", "-std=c++17", f"-I{INCLUDE}",
          f"-I{rocm}/include", "-D__HIP_PLATFORM_AMD__", f"-L{PKG_DIR}", "-lpagedkv",
          f"-L{rocm}/lib", "-lamdhip64", "-Wl,-rpath,$ORIGIN/../paged_kv_cache_244_amd"])
    os.replace(tmp, C_ABI_TEST_BIN)
    return C_ABI_TEST_BIN


if __name__ == "__main__":
    build(timeline="--timeline" in sys.argv[1:])
    sys.exit(0)
