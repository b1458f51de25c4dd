"""Build the HIP library ``libssd_scan.so`` in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("ssd_scan.hip", "sel_scan.hip", "trap_scan.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libssd_scan.so")

HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
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


def build(out: str = LIB, extra=()) -> str:
    """Compile the HIP sources into ``out`` (atomic replace)."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-o", tmp, *SRCS]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
