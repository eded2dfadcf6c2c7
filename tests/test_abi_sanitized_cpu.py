"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

``build_all`` compiles ``libdcptopk_host_sanitized.so``: the product's sources
with every host-side function (argument checks, span and overflow arithmetic,
workspace sizes, launch set-up) instrumented, and the product's device code.
Here every validation-only call of test_abi_cpu.py and of the plain-C consumer
runs against it, in processes that load the ASan runtime first; any invalid
read or write, signed overflow, misaligned access or other undefined behaviour
on those paths aborts the process and fails the test.  No GPU is touched: the
calls fail validation, or have nothing to do, before any HIP call.
"""
import os
import shutil
import subprocess
import sys

import pytest

from stable_top_selection_amd.build import INCLUDE, SANITIZED_LIB_PATH

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = "/opt/rocm/llvm/bin/clang"

pytestmark = pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not found")


def _asan_runtime() -> str:
    path = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("clang's ASan runtime not found")
    return path


def _env(**extra):
    env = dict(os.environ)
    # the HIP runtime keeps allocations until exit, which is not a leak of ours;
    # every other error ends the process at once
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra)
    return env


def test_sanitized_build_is_instrumented():
    """The build calls into both runtimes (so the checks below are live)."""
    assert os.path.exists(SANITIZED_LIB_PATH), "build the libraries first (python -m stable_top_selection_amd.build)"
    undefined = subprocess.run(["nm", "-D", "--undefined-only", SANITIZED_LIB_PATH], capture_output=True,
                               text=True).stdout
    assert "__asan_report_load" in undefined or "__asan_load" in undefined
    assert "__ubsan_handle_" in undefined


def test_abi_checks_under_sanitizers():
    """test_abi_cpu.py, loading the sanitized library instead of the product."""
    assert os.path.exists(SANITIZED_LIB_PATH), "build the libraries first"
    env = _env(LD_PRELOAD=_asan_runtime(), DCPTOPK_ABI_TEST_LIB=SANITIZED_LIB_PATH)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi_cpu.py")], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout and "failed" not in r.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out


def test_plain_c_consumer_under_sanitizers(tmp_path):
    """tests/c_abi/abi_check.c built with clang's sanitizers and linked against
    the sanitized library."""
    assert os.path.exists(SANITIZED_LIB_PATH), "build the libraries first"
    if shutil.which(CLANG) is None:
        pytest.skip("clang not found")
    lib_dir = tmp_path / "lib"
    lib_dir.mkdir()
    # the consumer links -ldcptopk: give the sanitized build that name
    os.symlink(SANITIZED_LIB_PATH, lib_dir / "libdcptopk.so")
    exe = tmp_path / "abi_check"
    cmd = [CLANG, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}", "-I/opt/rocm/include",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", os.path.join(HERE, "c_abi", "abi_check.c"),
           f"-L{lib_dir}", "-ldcptopk", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=_env())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout
    assert r.stdout.count("ok  ") == 16
