"""Build ``libdcptopk.so`` (HIP for gfx950) in the package directory.

``python -m stable_top_selection_amd.build`` compiles every source in
``csrc/`` with hipcc.  No GPU is needed to build.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libdcptopk.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# the same library with every odd wave delayed after each workgroup barrier
# (DCPTOPK_RACE_STRESS), for the race-stress tests only
STRESS_LIB_PATH = os.path.join(PKG, "libdcptopk_race_stress.so")
STRESS_FLAGS = ["-DDCPTOPK_RACE_STRESS=1"]
# the same library with shader-clock stamps at the select kernel's phase
# boundaries (DCPTOPK_PHASE_STAMPS), for stable_top_selection_amd.phase_report
PHASES_LIB_PATH = os.path.join(PKG, "libdcptopk_phases.so")
PHASE_FLAGS = ["-DDCPTOPK_PHASE_STAMPS=1"]
# the same library with its host code (the C ABI's checks and launch set-up)
# built with AddressSanitizer and UndefinedBehaviorSanitizer; the device code
# is the product's.  Only the CPU tests load it, in a process that preloads the
# ASan runtime (tests/test_abi_sanitized_cpu.py).
SANITIZED_LIB_PATH = os.path.join(PKG, "libdcptopk_host_sanitized.so")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
# reference kernels for the select's roofline (an empty launch, and a bare read
# and write of the headline's bytes), not part of the library; timed by
# stable_top_selection_amd.floor_probe
FLOOR_LIB_PATH = os.path.join(PKG, "libdcptopk_floor.so")
FLOOR_SOURCES = [os.path.join(PKG, "probes", "floor.hip")]
# per-kernel register, scratch, occupancy and LDS figures of the last build,
# from the compiler's resource-usage remarks
RESOURCES_PATH = os.path.join(PKG, "libdcptopk.kernels.tsv")
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
    # per-kernel resource usage, recorded next to the library
    "-Rpass-analysis=kernel-resource-usage",
]

_RESOURCE_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes",
                    "Occupancy [waves/SIMD]": "waves_per_simd", "VGPRs Spill": "vgpr_spill",
                    "SGPRs Spill": "sgpr_spill", "LDS Size [bytes/block]": "lds_bytes"}


def parse_resource_remarks(text: str) -> dict[str, dict[str, int]]:
    """Kernel name -> resource figures, from hipcc's resource-usage remarks."""
    kernels: dict[str, dict[str, int]] = {}
    name = None
    for line in text.splitlines():
        if "remark:" not in line or "kernel-resource-usage" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass-analysis", 1)[0].strip()
        if body.startswith("Function Name:"):
            name = body.split(":", 1)[1].strip()
            kernels[name] = {}
        elif name is not None and ":" in body:
            key, value = (x.strip() for x in body.rsplit(":", 1))
            if key in _RESOURCE_FIELDS and value.isdigit():
                kernels[name][_RESOURCE_FIELDS[key]] = int(value)
    return kernels


def write_resources(kernels: dict[str, dict[str, int]], path: str = RESOURCES_PATH) -> None:
    cols = list(_RESOURCE_FIELDS.values())
    with open(path, "w") as f:
        f.write("kernel\t" + "\t".join(cols) + "\n")
        for name in sorted(kernels):
            f.write(name + "\t" + "\t".join(str(kernels[name].get(c, -1)) for c in cols) + "\n")


def read_resources(path: str = RESOURCES_PATH) -> dict[str, dict[str, int]]:
    with open(path) as f:
        header = f.readline().rstrip("\n").split("\t")[1:]
        return {p[0]: dict(zip(header, map(int, p[1:]))) for p in (ln.rstrip("\n").split("\t") for ln in f) if p[0]}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libdcptopk")
    return path


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str = LIB_PATH,
          srcs: list[str] | None = None) -> str:
    """Compile and link the library (or `srcs` into `out`); returns the path
    of the shared object."""
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", "-shared", *(srcs or sources()), "-o",
           out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    noise = "is not a recognized feature for this target"  # host pass of the packed-fp32 switch
    # drop the resource remarks and the source excerpts printed under them
    warnings = [ln for ln in res.stderr.splitlines()
                if ln.strip() and noise not in ln and "kernel-resource-usage" not in ln
                and not re.match(r"^\s*\d*\s*\|", ln)]
    if verbose and warnings:
        print("\n".join(warnings), file=sys.stderr)
    os.replace(out + ".tmp", out)
    if out == LIB_PATH:
        write_resources(parse_resource_remarks(res.stderr))
    return out


def build_all(verbose: bool = False) -> list[str]:
    """The four libraries (product, race-stress test build, phase-stamp build,
    host-sanitized build) and the roofline reference kernels, compiled
    concurrently."""
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(max_workers=5) as pool:
        main = pool.submit(build, verbose)
        stress = pool.submit(build, False, STRESS_FLAGS, STRESS_LIB_PATH)
        phases = pool.submit(build, False, PHASE_FLAGS, PHASES_LIB_PATH)
        sanitized = pool.submit(build, False, SANITIZE_FLAGS, SANITIZED_LIB_PATH)
        floor = pool.submit(build, False, None, FLOOR_LIB_PATH, FLOOR_SOURCES)
        return [main.result(), stress.result(), phases.result(), sanitized.result(), floor.result()]


if __name__ == "__main__":
    print("\n".join(build_all(verbose=True)))
