"""Compile librns_gemm.so (HIP for gfx950) in-tree with hipcc.

The library is plain HIP (no PyTorch types): ``csrc/rns_host.cpp`` holds the
C ABI and host logic; ``csrc/rns_split.hip``, ``csrc/rns_gemm.hip``, ``csrc/rns_crt.hip``,
``csrc/rns_garner.hip``, ``csrc/rns_enclose.hip`` and ``csrc/rns_solve.hip`` the
device kernels, with shared device helpers in
``csrc/rns_device.h``; ``csrc/rns_ratrec.cpp`` the host stage of the exact solve
(big integers through the system's libgmp.so.10, opened at run time);
``csrc/rns_sliced.hip`` products beyond the residue capacity by operand slices;
``csrc/rns_noalloc.hip`` the product with the workspace in a fixed device array;
``csrc/rns_skinny.hip`` the batched-residue step for skinny right-hand sides in one kernel;
``csrc/rns_probe.hip`` a measurement aid (the int8 matrix-core rate with no memory traffic).
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librns_gemm.so")
SOURCES = [os.path.join(CSRC, f) for f in ("rns_host.cpp", "rns_split.hip", "rns_gemm.hip", "rns_crt.hip", "rns_garner.hip",
                                                    "rns_enclose.hip", "rns_solve.hip", "rns_ratrec.cpp",
                                                    "rns_sliced.hip", "rns_noalloc.hip", "rns_skinny.hip",
                                                    "rns_probe.hip")]
HEADERS = [os.path.join(CSRC, "rns_internal.h"), os.path.join(CSRC, "rns_device.h"),
           os.path.join(os.path.dirname(HERE), "include", "rns_gemm.h"),
           os.path.join(os.path.dirname(HERE), "include", "rns_enclose.h"),
           os.path.join(os.path.dirname(HERE), "include", "rns_solve.h"),
           os.path.join(os.path.dirname(HERE), "include", "rns_sliced.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are disabled for all device code; the host pass
# warns that it does not know the feature, which is harmless.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Wall", "-Wno-unused-function", "-pthread",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    """Always recompiles; returns the library path."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
