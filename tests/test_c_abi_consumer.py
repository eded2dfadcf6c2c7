"""The C ABI from plain C: tests/c_abi/abi_check.c compiles with gcc against
include/libdcptopk.h, links libdcptopk.so and runs its validation-only calls
(no GPU needed)."""
import os
import shutil
import subprocess

import pytest

from stable_top_selection_amd.build import INCLUDE, LIB_PATH

HERE = os.path.dirname(os.path.abspath(__file__))
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_plain_c_consumer(tmp_path):
    assert os.path.exists(LIB_PATH), "build the library first"
    exe = tmp_path / "abi_check"
    lib_dir = os.path.dirname(LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}", f"-I{ROCM_INCLUDE}",
           os.path.join(HERE, "c_abi", "abi_check.c"), f"-L{lib_dir}", "-ldcptopk", f"-Wl,-rpath,{lib_dir}",
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout
    assert r.stdout.count("ok  ") == 16
