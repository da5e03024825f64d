"""Build libtsdf_hip.so, the gfx950 HIP library behind include/tsdf.h.

    python -m hash_table_amd.build

Compiles in-tree with hipcc (cross-compiles without a GPU).  Float flags:
no FMA contraction, correctly rounded f32 division and no denormal flushing,
so the band walk takes the same f32 decisions as any other IEEE
implementation of it; packed-fp32 instructions are disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libtsdf_hip.so")
SOURCES = [os.path.join(CSRC, n) for n in ("tsdf_kernels.hip", "tsdf_mesh.hip", "tsdf_capi.hip", "microbench.hip")]
HEADERS = [os.path.join(CSRC, "tsdf_device.hpp"), os.path.join(CSRC, "tsdf_kernels.hpp"), os.path.join(ROOT, "include", "tsdf.h"),
           os.path.join(ROOT, "include", "tsdf_microbench.h")]
ARCH = os.environ.get("TSDF_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(output: str = LIBRARY, extra_flags=(), verbose: bool = False) -> str:
    tmp = output + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    noise = [ln for ln in (proc.stdout + proc.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "warning generated" not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise))
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
