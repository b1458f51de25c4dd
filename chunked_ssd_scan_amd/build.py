"""Build the HIP library ``libssd_scan.so`` in-tree with hipcc for gfx950.

Each source compiles to its own object (in parallel), then one link step makes
the shared library. Objects live in ``_build/`` next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC_NAMES = ("ssd_scan.hip", "ssd_walk_bf16.hip", "ssd_walk_f32.hip", "ssd_cols_bf16.hip",
             "ssd_cols_f32.hip", "sel_scan.hip", "trap_scan.hip", "moments.hip",
             "ssd_backward.hip")
SRCS = [os.path.join(HERE, "csrc", f) for f in SRC_NAMES]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libssd_scan.so")
OBJDIR = os.path.join(HERE, "_build")

HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs: the running state is also scaled by
    # VALU every tile, and AGPR copies would cost more than they save
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _compile(src: str, obj: str, extra) -> None:
    tmp = obj + f".tmp{os.getpid()}"
    subprocess.run([hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-c", "-o", tmp, src], check=True)
    os.replace(tmp, obj)


def build(out: str = LIB, extra=()) -> str:
    """Compile the HIP sources into ``out`` (atomic replace)."""
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.splitext(n)[0] + ".o") for n in SRC_NAMES]
    with ThreadPoolExecutor(max_workers=len(SRCS)) as pool:
        for f in [pool.submit(_compile, s, o, tuple(extra)) for s, o in zip(SRCS, objs)]:
            f.result()
    tmp = out + f".tmp{os.getpid()}"
    subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                   check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
