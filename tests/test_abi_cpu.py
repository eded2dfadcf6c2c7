"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and its host-side checks return the documented status codes without
enqueueing anything (no GPU is touched: every call here fails validation, or
has rows == 0, before any HIP call)."""
import ctypes
import os
import subprocess

import pytest

from oracle import stable_topk as O
from stable_top_selection_amd import binding as B
from stable_top_selection_amd.build import LIB_PATH, STRESS_LIB_PATH

# the library under test: the product build, or another build of the same
# sources named by DCPTOPK_ABI_TEST_LIB (test_abi_sanitized_cpu.py runs this
# module on the host-sanitized build)
ABI_LIB = os.environ.get("DCPTOPK_ABI_TEST_LIB", LIB_PATH)

P = ctypes.c_void_p
DEV_A = 0x7F0000000000  # fake, 256-byte aligned device addresses: never dereferenced
DEV_B = 0x7F0010000000


@pytest.fixture(scope="module")
def lib():
    return B.load_library() if ABI_LIB == LIB_PATH else B.open_library(ABI_LIB)


def test_exports_every_header_function(lib):
    names = B.header_functions()
    assert set(names) == {"dcp_topk_pack", "dcp_topk_select", "dcp_topk_merge_workspace_bytes",
                          "dcp_topk_merge_chunked", "dcp_topk_merge_chunked_static", "dcp_topk_merge_fused",
                          "dcp_topk_local", "dcp_topk_status_string", "dcp_topk_select_split",
                          "dcp_topk_select_split_workspace_bytes"}
    for n in names:
        assert hasattr(lib, n), n
    exported = subprocess.run(["nm", "-D", "--defined-only", ABI_LIB], capture_output=True, text=True).stdout
    public = sorted(line.split()[-1] for line in exported.splitlines() if " T dcp_topk_" in line)
    assert public == names


def test_race_stress_build_exports_the_same_functions():
    """The race-stress build (the GPU race tests load it) is the same library
    with delayed waves: same entry points, same signatures."""
    stress = B.open_library(STRESS_LIB_PATH)
    names = B.header_functions()
    for n in names:
        assert hasattr(stress, n), n
    exported = subprocess.run(["nm", "-D", "--defined-only", STRESS_LIB_PATH], capture_output=True, text=True).stdout
    assert sorted(line.split()[-1] for line in exported.splitlines() if " T dcp_topk_" in line) == names
    assert stress.dcp_topk_status_string(0) == b"ok"


def test_status_strings(lib):
    st = lambda code: lib.dcp_topk_status_string(code).decode()  # noqa: E731
    assert st(0) == "ok"
    assert "invalid" in st(-1)
    assert "unsupported" in st(-2)
    assert "workspace" in st(-3)
    assert "HIP" in st(-4)
    assert "static scratch" in st(-5)
    assert st(99) == "unknown status"
    assert B.status_string(-1) == st(-1)


@pytest.mark.parametrize("rows,dcp,local_k", [(0, 4, 2048), (1, 4, 2048), (1024, 4, 2048), (1025, 4, 2048),
                                              (8192, 4, 2048), (5, 3, 7), (-1, 4, 2048)])
def test_workspace_bytes_match_oracle(lib, rows, dcp, local_k):
    want = O.merge_workspace_bytes(rows, dcp, local_k) if rows >= 0 else 0
    assert lib.dcp_topk_merge_workspace_bytes(rows, dcp, local_k) == want


def test_workspace_bytes_that_do_not_fit_a_size_t(lib):
    """1024 rows of 2^62 candidates need 2^75 bytes: no size, so 0 (the merge
    rejects such a shape as unsupported before it looks at the workspace)."""
    big = 2**31 - 1
    assert lib.dcp_topk_merge_workspace_bytes(1024, big, big) == 0
    assert lib.dcp_topk_merge_workspace_bytes(big, 16, big) == O.merge_workspace_bytes(big, 16, big)


def test_select_argument_checks(lib):
    s = lib.dcp_topk_select
    assert s(None, 0, 8192, 2048, None, None) == B.OK  # no rows: nothing to do
    assert s(None, 1, 8192, 2048, P(DEV_B), None) == B.EINVAL  # null input
    assert s(P(DEV_A), 1, 8192, 2048, None, None) == B.EINVAL  # null output
    assert s(P(DEV_A), 1, 8192, 0, P(DEV_B), None) == B.EINVAL  # k < 1
    assert s(P(DEV_A), -1, 8192, 1, P(DEV_B), None) == B.EINVAL
    assert s(P(DEV_A), 1, -5, 1, P(DEV_B), None) == B.EINVAL
    assert s(P(DEV_A + 4), 1, 64, 1, P(DEV_B), None) == B.EINVAL  # misaligned input
    assert s(P(DEV_A), 1, 64, 1, P(DEV_B + 2), None) == B.EINVAL  # misaligned output
    assert s(P(DEV_A), 1, 16385, 1, P(DEV_B), None) == B.EUNSUPPORTED
    assert s(P(DEV_A), 1, 64, 16385, P(DEV_B), None) == B.EUNSUPPORTED  # k past the limit
    # output overlapping the input: row 1 of the input is the output
    assert s(P(DEV_A), 4, 64, 16, P(DEV_A + 64 * 8), None) == B.EINVAL


def test_row_limit(lib):
    """Past DCP_TOPK_MAX_ROWS rows every single-launch entry point returns
    DCP_TOPK_EUNSUPPORTED before any launch (the grid's thread count is a
    32-bit number); the chunked merge takes any row count."""
    big = B.MAX_ROWS + 1
    far = 0x7F8000000000  # fake outputs well past the fake inputs' spans
    assert lib.dcp_topk_select(P(DEV_A), big, 1, 1, P(far), None) == B.EUNSUPPORTED
    assert lib.dcp_topk_select(P(DEV_A), big, -1, 1, P(far), None) == B.EINVAL  # checked first
    ws = P(far + 0x100000000)
    assert lib.dcp_topk_select_split(P(DEV_A), big, 64, 1, 2, ws, 1 << 30, P(far), None) == B.EUNSUPPORTED
    assert lib.dcp_topk_pack(P(DEV_A), P(DEV_A + 0x100000000), 1, P(DEV_A + 0x200000000), 0, big, 1, P(far), 1,
                             None) == B.EUNSUPPORTED
    ranks = _rank_arrays(1)
    assert lib.dcp_topk_merge_fused(*ranks, 1, big, 64, 1, P(far), None) == B.EUNSUPPORTED
    assert lib.dcp_topk_local(P(DEV_A), 1, None, big, 1, 1, P(far), P(far + 0x100000000), 1, None) == B.EUNSUPPORTED
    # the limit itself is accepted by the checks: rows == 0 aside, a call that
    # passes every check would launch, so only a check that fails later is used
    assert lib.dcp_topk_select(P(DEV_A), B.MAX_ROWS, 1, 1, P(DEV_A + 8), None) == B.EINVAL  # overlap, not the limit


def test_pack_argument_checks(lib):
    p = lib.dcp_topk_pack
    a, b, c, d = P(DEV_A), P(DEV_A + 0x100000), P(DEV_A + 0x200000), P(DEV_B)
    assert p(None, None, 0, None, 0, 0, 16, None, 0, None) == B.OK  # no rows
    assert p(a, b, 16, c, 0, 4, 0, d, 16, None) == B.OK  # no columns
    assert p(None, b, 16, c, 0, 4, 16, d, 16, None) == B.EINVAL
    assert p(a, b, 15, c, 0, 4, 16, d, 16, None) == B.EINVAL  # source stride < local_k
    assert p(a, b, 16, c, 0, 4, 16, d, 15, None) == B.EINVAL  # dst stride < local_k
    assert p(a, b, 16, c, 0, 4, 16, P(DEV_B + 4), 16, None) == B.EINVAL  # dst misaligned
    assert p(a, b, 16, c, 0, 4, 16, b, 16, None) == B.EINVAL  # dst overlaps the indices
    assert p(a, b, 16, c, 0, -4, 16, d, 16, None) == B.EINVAL


def test_merge_argument_checks(lib):
    m = lib.dcp_topk_merge_chunked
    arr = ctypes.c_void_p * 2
    sc = arr(DEV_A, DEV_A + 0x1000000)
    ix = arr(DEV_A + 0x2000000, DEV_A + 0x3000000)
    rs = arr(DEV_A + 0x4000000, DEV_A + 0x5000000)
    offs = (ctypes.c_int32 * 2)(0, 1000)
    ws_need = lib.dcp_topk_merge_workspace_bytes(64, 2, 128)
    cast = lambda x: ctypes.cast(x, P)  # noqa: E731
    args = lambda ws, wsb, out, dcp=2, rows=64, lk=128, k=64: (  # noqa: E731
        cast(sc), cast(ix), cast(rs), cast(offs), dcp, rows, lk, k, P(ws), wsb, P(out), None)
    assert m(*args(DEV_B, ws_need, DEV_B + 0x1000000, rows=0)) == B.OK
    assert m(*args(DEV_B, ws_need, DEV_B + 0x1000000, dcp=0)) == B.EINVAL
    assert m(*args(DEV_B, ws_need, DEV_B + 0x1000000, k=0)) == B.EINVAL
    assert m(*args(DEV_B, ws_need, DEV_B + 0x1000000, lk=16384)) == B.EUNSUPPORTED
    assert m(*args(DEV_B, ws_need - 1, DEV_B + 0x1000000)) == B.EWORKSPACE
    assert m(*args(DEV_B + 64, ws_need, DEV_B + 0x1000000)) == B.EWORKSPACE  # not 256-byte aligned
    assert m(*args(None, ws_need, DEV_B + 0x1000000)) == B.EWORKSPACE
    assert m(*args(DEV_B, ws_need, DEV_B + 256)) == B.EINVAL  # out overlaps the workspace
    assert m(*args(DEV_B, ws_need, DEV_A + 0x2000000)) == B.EINVAL  # out overlaps rank 0's indices
    assert m(*args(DEV_A + 0x4000000, ws_need, DEV_B)) == B.EINVAL  # workspace overlaps row starts
    assert m(None, cast(ix), cast(rs), cast(offs), 2, 64, 128, 64, P(DEV_B), ws_need, P(DEV_B + 0x1000000),
             None) == B.EINVAL


def _rank_arrays(n, base=DEV_A):
    arr = ctypes.c_void_p * n
    sc = arr(*[base + r * 0x1000000 for r in range(n)])
    ix = arr(*[base + 0x40000000 + r * 0x1000000 for r in range(n)])
    rs = arr(*[base + 0x80000000 + r * 0x1000000 for r in range(n)])
    offs = (ctypes.c_int32 * n)(*[r * 1000 for r in range(n)])
    return [ctypes.cast(x, P) for x in (sc, ix, rs, offs)]


def test_merge_fused_argument_checks(lib):
    f = lib.dcp_topk_merge_fused
    ok = _rank_arrays(2)
    args = lambda out, dcp=2, rows=64, lk=128, k=64, ranks=ok: (*ranks, dcp, rows, lk, k, P(out), None)  # noqa: E731
    assert f(*args(DEV_B, rows=0)) == B.OK
    assert f(*args(DEV_B, dcp=0)) == B.EINVAL
    assert f(*args(DEV_B, k=0)) == B.EINVAL
    assert f(*args(DEV_B, rows=-1)) == B.EINVAL
    assert f(*args(DEV_B, lk=100)) == B.EUNSUPPORTED  # local_k not a multiple of 64
    assert f(*args(DEV_B, k=16385)) == B.EUNSUPPORTED
    many = _rank_arrays(17)
    assert f(*args(DEV_B, dcp=17, ranks=many)) == B.EUNSUPPORTED
    three = _rank_arrays(3)
    assert f(*args(DEV_B, dcp=3, lk=8192, ranks=three)) == B.EUNSUPPORTED  # 24576 candidates
    assert f(*args(None)) == B.EINVAL
    assert f(*args(DEV_B + 4)) == B.EINVAL  # output not 8-byte aligned
    assert f(*args(DEV_A + 0x40000000)) == B.EINVAL  # output overlaps rank 0's indices
    assert f(*args(DEV_A + 0x81000000)) == B.EINVAL  # output overlaps rank 1's row starts
    null_rank = _rank_arrays(2)
    ctypes.cast(null_rank[0], ctypes.POINTER(ctypes.c_void_p))[1] = None
    assert f(*args(DEV_B, ranks=null_rank)) == B.EINVAL
    assert f(None, ok[1], ok[2], ok[3], 2, 64, 128, 64, P(DEV_B), None) == B.EINVAL


def test_local_argument_checks(lib):
    loc = lib.dcp_topk_local
    a, lens, os_, oi = DEV_A, DEV_A + 0x1000000, DEV_B, DEV_B + 0x1000000
    args = lambda s=a, stride=4096, ln=None, rows=64, cols=4096, k=2048, o1=os_, o2=oi, ostride=2048: (  # noqa: E731
        P(s), stride, P(ln), rows, cols, k, P(o1), P(o2), ostride, None)
    assert loc(*args(rows=0)) == B.OK
    assert loc(*args(rows=-1)) == B.EINVAL
    assert loc(*args(k=0)) == B.EINVAL
    assert loc(*args(cols=-1)) == B.EINVAL
    assert loc(*args(cols=16385, stride=16385)) == B.EUNSUPPORTED
    assert loc(*args(k=16385, ostride=16385)) == B.EUNSUPPORTED
    assert loc(*args(s=None)) == B.EINVAL
    assert loc(*args(o1=None)) == B.EINVAL
    assert loc(*args(o2=None)) == B.EINVAL
    assert loc(*args(stride=4095)) == B.EINVAL  # row stride narrower than the row
    assert loc(*args(ostride=2047)) == B.EINVAL
    assert loc(*args(s=a + 2)) == B.EINVAL  # misaligned scores
    assert loc(*args(o2=oi + 1)) == B.EINVAL  # misaligned index output
    assert loc(*args(ln=lens + 2)) == B.EINVAL  # misaligned lengths
    assert loc(*args(o2=os_ + 4)) == B.EINVAL  # the two outputs overlap
    assert loc(*args(o1=a + 4096 * 4)) == B.EINVAL  # score output inside the scores
    assert loc(*args(ln=oi + 64)) == B.EINVAL  # lengths inside the index output


def _split_bytes(rows, num_cand, parts):
    """The split workspace as the header describes it: four regions, each
    rounded up to 256 bytes."""
    up = lambda x: (x + 255) // 256 * 256
    return up(rows * 16) + up(rows * parts * 8224) + up(rows * num_cand * 8) + up(rows * num_cand * 4)


@pytest.mark.parametrize("rows,num_cand,parts", [(0, 8192, 4), (1, 8192, 1), (16, 8192, 4), (64, 8192, 8),
                                                 (3, 1000, 3), (5, 16384, 2), (1, 0, 2)])
def test_split_workspace_bytes(lib, rows, num_cand, parts):
    assert lib.dcp_topk_select_split_workspace_bytes(rows, num_cand, parts) == _split_bytes(rows, num_cand, parts)


def test_split_workspace_bytes_rejects_bad_arguments(lib):
    f = lib.dcp_topk_select_split_workspace_bytes
    assert f(-1, 8192, 4) == 0 and f(1, -1, 4) == 0 and f(1, 8192, 0) == 0 and f(1, 8192, 9) == 0
    assert f(1, 16385, 4) == 0 and f(2**31 - 1, 2**31 - 1, 8) == 0  # past DCP_TOPK_MAX_CANDIDATES


def test_select_split_argument_checks(lib):
    s = lib.dcp_topk_select_split
    ws = 0x7F0020000000
    need = _split_bytes(16, 8192, 4)
    assert s(None, 0, 8192, 2048, 4, None, 0, None, None) == B.OK  # no rows
    assert s(None, 16, 8192, 2048, 4, P(ws), need, P(DEV_B), None) == B.EINVAL  # null input
    assert s(P(DEV_A), 16, 8192, 0, 4, P(ws), need, P(DEV_B), None) == B.EINVAL  # k < 1
    assert s(P(DEV_A), 16, 8192, 2048, 0, P(ws), need, P(DEV_B), None) == B.EUNSUPPORTED  # parts < 1
    assert s(P(DEV_A), 16, 8192, 2048, 9, P(ws), need, P(DEV_B), None) == B.EUNSUPPORTED  # parts > 8
    assert s(P(DEV_A), 1, 16384, 2048, 1, P(ws), 1 << 30, P(DEV_B), None) == B.EUNSUPPORTED  # slice > 8192
    assert s(P(DEV_A), 16, 8192, 2048, 4, None, need, P(DEV_B), None) == B.EWORKSPACE
    assert s(P(DEV_A), 16, 8192, 2048, 4, P(ws + 8), need, P(DEV_B), None) == B.EWORKSPACE  # misaligned
    assert s(P(DEV_A), 16, 8192, 2048, 4, P(ws), need - 1, P(DEV_B), None) == B.EWORKSPACE  # short
    # workspace overlapping the input or the output
    assert s(P(DEV_A), 16, 8192, 2048, 4, P(DEV_A + 4096), need, P(DEV_B), None) == B.EINVAL
    assert s(P(DEV_A), 16, 8192, 2048, 4, P(DEV_B - 256), need, P(DEV_B), None) == B.EINVAL
