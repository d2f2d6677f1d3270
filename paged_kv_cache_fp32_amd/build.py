"""Ahead-of-time build of the HIP library ``libdsv4_c128.so`` for gfx950.

    python -m paged_kv_cache_fp32_amd.build

Compiles the kernel and the C ABI with hipcc into the package directory, so
the shared library travels with the source tree.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdsv4_c128.so")
SOURCES = [os.path.join(CSRC, "c128_kernel.hip"), os.path.join(CSRC, "c128_schedules.hip"),
           os.path.join(CSRC, "c4_kernel.hip"), os.path.join(CSRC, "indexer_kernel.hip"),
           os.path.join(CSRC, "c128_abi.cpp")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(force: bool = True, verbose: bool = False) -> str:
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
