"""The roofline reference kernels (stable_top_selection_amd.floor_probe) on
the CPU: a library of their own, exporting only their four entry points, whose
host checks reject bad launches without touching a GPU."""
import ctypes
import subprocess

from stable_top_selection_amd import floor_probe as F
from stable_top_selection_amd.build import FLOOR_LIB_PATH

P = ctypes.c_void_p
DEV_A = 0x7F0000000000  # fake, 256-byte aligned device addresses: never dereferenced
DEV_B = 0x7F0010000000


def test_floor_reference_kernels_build():
    """Four exported entry points; the select's per-row bytes; the host
    checks; the launch counts of the timed graphs."""
    exported = subprocess.run(["nm", "-D", "--defined-only", FLOOR_LIB_PATH], capture_output=True, text=True).stdout
    names = sorted(line.split()[-1] for line in exported.splitlines() if " T " in line)
    assert names == ["floor_empty", "floor_row_read_bytes", "floor_row_write_bytes", "floor_stream"]
    flib = ctypes.CDLL(FLOOR_LIB_PATH)
    flib.floor_row_read_bytes.restype = ctypes.c_int64
    flib.floor_row_write_bytes.restype = ctypes.c_int64
    assert flib.floor_row_read_bytes() == 8192 * 8 and flib.floor_row_write_bytes() == 2048 * 8
    flib.floor_stream.argtypes = [P, P, P, ctypes.c_int32, P]
    assert flib.floor_stream(P(DEV_A + 8), None, P(DEV_B), 256, None) == -1  # misaligned: nothing launched
    assert flib.floor_stream(P(DEV_A), None, P(DEV_B), 0, None) == -1
    flib.floor_empty.argtypes = [ctypes.c_int32, ctypes.c_int32, P]
    assert flib.floor_empty(256, 2048, None) == -1 and flib.floor_empty(0, 64, None) == -1
    assert F.launches(1) == 200 and F.launches(36) == 216 and F.launches(200) == 200
    assert F.EMPTY_SHAPES[0] == (256, 512)  # the headline's launch shape
