"""Register, scratch and occupancy budgets of the built kernels, from the
compiler's resource-usage remarks that every build records next to the
library.

The many-row launches (the fused merge over a prefill batch, the chunked
merge, the local top-K over many rows, with or without per-row lengths) rely
on two 512-thread workgroups sharing a CU, so that one row's selection
overlaps the next row's loads: the kernels they use must stay within 128
VGPRs (4 waves per SIMD).  Losing that halves their throughput with no change
in results, which no parity test would notice.
"""
import os
import re

import pytest

from stable_top_selection_amd import build as BLD

pytestmark = pytest.mark.skipif(not os.path.exists(BLD.RESOURCES_PATH),
                                reason="library not built (run __graft_entry__.build())")

SELECT = re.compile(r"stable_topk_kernelILi(\d+)ELi(\d+)ELi(\d+)ELb([01])ENS0_\d+(\w+?Source)")

def _select_kernels():
    out = []
    for name, r in BLD.read_resources().items():
        m = SELECT.search(name)
        if m:
            block, vec, n, full, source = int(m[1]), int(m[2]), int(m[3]), m[4] == "1", m[5]
            out.append((name, block, vec, n, full, source, r))
    return out


def test_every_kernel_reported():
    kernels = BLD.read_resources()
    assert sum(1 for n in kernels if "pack_kernel" in n) == 4  # {vector, scalar} x {256, 512} threads
    assert len(_select_kernels()) >= 90


def test_every_8_and_16_item_kernel_fits_two_workgroups_per_cu():
    """Every 512-thread kernel of 8 or 16 items per thread, full-row or
    partial-row (per-row lengths, candidate counts that are not a multiple of
    the block), of every source: at most 128 VGPRs (4 waves per SIMD) and
    LDS for two workgroups per CU."""
    seen = set()
    for name, block, vec, n, full, source, r in _select_kernels():
        if block == 512 and n in (8, 16):
            seen.add((source, vec, n, full))
            assert r["waves_per_simd"] >= 4, f"{name}: {r['vgprs']} VGPRs, {r['waves_per_simd']} waves per SIMD"
            assert 2 * r["lds_bytes"] <= 160 * 1024, f"{name}: {r['lds_bytes']} B of LDS per workgroup"
    expected = {(src, vec, n, full) for src in ("GatheredSource", "RankSource", "DenseSource") for vec in (1, 2, 4)
                for n in (8, 16) for full in (False, True) if not (src == "GatheredSource" and vec == 4)}
    assert expected <= seen, sorted(expected - seen)


def test_no_scratch_in_any_kernel():
    """No kernel spills to memory: every select instance the entry points can
    launch (up to 32 items per thread, so every row of up to 16384
    candidates, partial rows included) and both pack kernels."""
    kernels = _select_kernels()
    assert any(n == 32 and not full and source == "RankSource" for _, _, _, n, full, source, _ in kernels)
    for name, block, vec, n, full, source, r in kernels:
        assert r["scratch_bytes"] == 0 and r["vgpr_spill"] == 0, f"{name}: {r}"
    for name, r in BLD.read_resources().items():
        if "pack_kernel" in name:
            assert r["scratch_bytes"] == 0, f"{name}: {r}"


def test_remark_parser():
    text = ("a.hip:1:1: remark: Function Name: kern [-Rpass-analysis=kernel-resource-usage]\n"
            "a.hip:1:1: remark:     VGPRs: 113 [-Rpass-analysis=kernel-resource-usage]\n"
            "a.hip:1:1: remark:     Occupancy [waves/SIMD]: 4 [-Rpass-analysis=kernel-resource-usage]\n"
            "a.hip:1:1: remark:     LDS Size [bytes/block]: 77680 [-Rpass-analysis=kernel-resource-usage]\n"
            "    1 | int x;\n")
    assert BLD.parse_resource_remarks(text) == {"kern": {"vgprs": 113, "waves_per_simd": 4, "lds_bytes": 77680}}


def test_1024_thread_kernels_fit_the_simds():
    """Rows of more than 8192 candidates (partial gathered rows, every fused
    and dense row) run 1024 threads x 16 items: a workgroup of 16 waves needs
    4 waves per SIMD (at most 128 VGPRs) to launch at all, and its LDS must fit
    one CU."""
    seen = set()
    for name, block, vec, n, full, source, r in _select_kernels():
        if block == 1024:
            seen.add((source, vec, full))
            assert n == 16, name
            assert r["waves_per_simd"] >= 4, f"{name}: {r['vgprs']} VGPRs"
            assert r["lds_bytes"] <= 160 * 1024, f"{name}: {r['lds_bytes']} B of LDS"
    expected = {("GatheredSource", 1, False), ("GatheredSource", 2, False), ("RankSource", 4, False),
                ("RankSource", 4, True), ("DenseSource", 4, False), ("DenseSource", 4, True)}
    assert expected <= seen, sorted(expected - seen)
