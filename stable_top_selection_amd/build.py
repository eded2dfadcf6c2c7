"""Build ``libdcptopk.so`` (HIP for gfx950) in the package directory.

``python -m stable_top_selection_amd.build`` compiles every source in
``csrc/`` with hipcc.  No GPU is needed to build.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libdcptopk.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-result",
    # no packed fp32 instructions anywhere (the library does no fp32 arithmetic
    # at all; this keeps the compiler from forming them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libdcptopk")
    return path


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str = LIB_PATH) -> str:
    """Compile and link the library; returns the path of the shared object."""
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", "-shared", *sources(), "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    noise = "is not a recognized feature for this target"  # host pass of the packed-fp32 switch
    warnings = [ln for ln in res.stderr.splitlines() if ln.strip() and noise not in ln]
    if verbose and warnings:
        print("\n".join(warnings), file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
