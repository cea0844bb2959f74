"""Build libgemm355.so in-tree with hipcc for gfx950 (no GPU needed to compile)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libgemm355.so")
SOURCES = [os.path.join(CSRC, "gemm355.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("common.hpp", "gemm_bf16.hpp", "gemm_bf16_small.hpp", "gemm_bf16_small_long.hpp", "gemm_bf16_splitk.hpp",
                                           "gemm_fp4.hpp", "fp4_decode.hpp", "gemm_mxfp4.hpp", "schedule.hpp")] + \
    [os.path.join(INCLUDE, "gemm355.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # the LDS copies clobber m0 on purpose (the compiler uses m0 nowhere else)
    "-Wno-inline-asm",
    # packed FP32 instructions stay off: the compiler must not form them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source of the library into LIB_PATH. Always recompiles."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "unknown target feature")
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if l and not any(n in l for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, "\n".join(msgs)))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def stale() -> bool:
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
