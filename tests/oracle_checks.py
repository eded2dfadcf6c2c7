"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Every check calls the oracle through ``oracle.stable_topk`` attributes at call
time, so ``test_oracle_mutants.py`` can plant a mistake in the oracle and see
that at least one check fails.  None of these checks re-types the oracle's own
formulas:

* ``brute_*``      pure-Python O(C^2) rank counting under IEEE 754 totalOrder
                   written from its definition (no bit tricks), then the pages'
                   tie rule (lowest id) and the stable rule (lowest position).
* library pins     ``torch.topk`` / ``np.argpartition`` on rows with distinct
                   scores; ``np.sort`` of the ids on all-tie rows.
* invariants       count, dominance, candidate-position order, padding.
* printed figures  the merge-scratch sizes printed on PR #59367 (Purpose),
                   stored in ``tests/golden/pages_memory_figures.json``.
"""
from __future__ import annotations

import itertools
import json
import math
import os
import struct

import numpy as np

from oracle import stable_topk as O
from stable_top_selection_amd import workloads as W

INT32_MAX = 2**31 - 1
PAD_BITS = 0xFF800000
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# brute force, written from definitions only
# ----------------------------------------------------------------------------
def _f32(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]


def total_order(bits: int):
    """Position of an fp32 bit pattern in IEEE 754 totalOrder as a tuple.

    -NaN (larger payload lower) < -inf < ... < -0 < +0 < ... < +inf < +NaN
    (larger payload higher).
    """
    x = _f32(bits)
    negative = (bits >> 31) & 1
    if math.isnan(x):
        payload = bits & 0x7FFFFF
        return (-1, -payload, 0) if negative else (1, payload, 0)
    return (0, x, 0 if negative else 1)


def _beats(a, b) -> bool:
    """Candidate a = (score bits, id, position) is ranked before b."""
    ta, tb = total_order(a[0]), total_order(b[0])
    if ta != tb:
        return ta > tb
    ua, ub = a[1] & 0xFFFFFFFF, b[1] & 0xFFFFFFFF
    if ua != ub:
        return ua < ub  # lowest global token id first
    return a[2] < b[2]  # lowest position first


def brute_select_row(bits, ids, k):
    """One row: returns (out score bits, out ids) as python lists of length k."""
    cands = [(int(bits[p]) & 0xFFFFFFFF, int(ids[p]), p) for p in range(len(bits))]
    chosen = []
    for c in cands:
        rank = sum(1 for d in cands if d is not c and _beats(d, c))
        if rank < k:
            chosen.append(c)
    chosen.sort(key=lambda c: c[2])
    out_bits = [c[0] for c in chosen] + [PAD_BITS] * (k - len(chosen))
    out_ids = [c[1] for c in chosen] + [INT32_MAX] * (k - len(chosen))
    return out_bits, out_ids


def _oracle_bits(scores, ids, k):
    s, i = O.select(scores, ids, k)
    return np.asarray(s, np.float32).view(np.uint32), np.asarray(i, np.int32)


def _assert_rows_match_brute(bits_rows, id_rows, k):
    bits_rows = np.asarray(bits_rows, np.uint32)
    id_rows = np.asarray(id_rows, np.int32)
    ob, oi = _oracle_bits(bits_rows.view(np.float32), id_rows, k)
    for r in range(bits_rows.shape[0]):
        eb, ei = brute_select_row(bits_rows[r], id_rows[r], k)
        assert [int(x) for x in ob[r]] == eb, f"row {r} k={k}: scores differ"
        assert [int(x) for x in oi[r]] == ei, f"row {r} k={k}: ids differ"


# ----------------------------------------------------------------------------
# checks
# ----------------------------------------------------------------------------
FINITE_LADDER = [
    0xFFFFFFFF,  # -NaN, largest payload
    0xFFC00000,  # -qNaN
    0xFF800001,  # -sNaN, smallest payload
    0xFF800000,  # -inf
    0xFF7FFFFF,  # -max
    0xBF800000,  # -1
    0x80800000,  # -min normal
    0x80000001,  # -min subnormal
    0x80000000,  # -0
    0x00000000,  # +0
    0x00000001,  # +min subnormal
    0x3F800000,  # +1
    0x7F7FFFFF,  # +max
    0x7F800000,  # +inf
    0x7F800001,  # +sNaN, smallest payload
    0x7FC00000,  # +qNaN
    0x7FFFFFFF,  # +NaN, largest payload
]


def check_score_key_ladder():
    """Keys must rise strictly along the totalOrder ladder of special values."""
    for lo, hi in zip(FINITE_LADDER, FINITE_LADDER[1:]):
        assert total_order(lo) < total_order(hi)  # the ladder itself is ordered
    keys = O.score_key(np.array(FINITE_LADDER, dtype=np.uint32).view(np.float32))
    assert np.all(np.diff(keys.astype(np.int64)) > 0), keys


def check_score_key_orders_like_floats(seed=0, n=200_000):
    """For non-NaN floats, comparing keys equals comparing floats (IEEE <),
    except that -0 sorts below +0."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    a, b = f[: len(f) // 2], f[len(f) // 2: 2 * (len(f) // 2)]
    ka, kb = O.score_key(a), O.score_key(b)
    lt = a < b
    gt = a > b
    assert np.array_equal(ka < kb, lt | ((a == b) & np.signbit(a) & ~np.signbit(b)))
    assert np.array_equal(ka > kb, gt | ((a == b) & ~np.signbit(a) & np.signbit(b)))
    # sorting by key reproduces numpy's float sort (values)
    vals = rng.standard_normal(10_000).astype(np.float32) * np.float32(1e3)
    assert np.array_equal(vals[np.argsort(O.score_key(vals), kind="stable")], np.sort(vals))


def check_exhaustive_tiny_rows():
    """Every row of 4 candidates over a 6-pair alphabet (including full
    duplicates, +-0, +-inf and padding), every K in 1..5, against brute force."""
    alphabet = [
        (0x3F800000, 5),  # 1.0, id 5
        (0x3F800000, 3),  # 1.0, id 3
        (0x80000000, 7),  # -0.0, id 7
        (0x00000000, 7),  # +0.0, id 7
        (0x7F800000, 1),  # +inf, id 1
        (PAD_BITS, INT32_MAX),  # padding
    ]
    rows = list(itertools.product(alphabet, repeat=4))
    bits = np.array([[c[0] for c in r] for r in rows], dtype=np.uint32)
    ids = np.array([[c[1] for c in r] for r in rows], dtype=np.int32)
    for k in range(1, 6):
        _assert_rows_match_brute(bits, ids, k)


def check_random_rows_with_specials(seed=1):
    """Random rows (C up to 48) with NaNs, +-0, +-inf, repeated scores and
    repeated (score, id) pairs, against brute force."""
    rng = np.random.default_rng(seed)
    specials = np.array(FINITE_LADDER + [0x40000000, 0xC0000000, 0x3F800000], dtype=np.uint32)
    for trial in range(60):
        c = int(rng.integers(1, 49))
        rows = 3
        pick = rng.integers(0, len(specials), size=(rows, c))
        bits = specials[pick]
        mix = rng.random((rows, c)) < 0.4
        bits = np.where(mix, rng.integers(0, 2**32, size=(rows, c), dtype=np.uint64).astype(np.uint32), bits)
        ids = rng.integers(0, 6, size=(rows, c)).astype(np.int32)
        ids[rng.random((rows, c)) < 0.1] = INT32_MAX
        k = int(rng.integers(1, c + 3))
        _assert_rows_match_brute(bits, ids, k)


def check_configs_tiny_against_brute():
    """The tiny workload (4 rows x 256, K 64) against brute force."""
    g = W.tiny()
    _assert_rows_match_brute(g.scores.view(np.uint32), g.ids, g.k)


def check_distinct_scores_match_library_topk(seed=2):
    """Distinct scores: the selected set is the library's top-K set
    (torch.topk and numpy.argpartition), emitted in position order."""
    import torch

    rng = np.random.default_rng(seed)
    for c, k in [(256, 64), (1000, 1), (1000, 999), (8192, 2048)]:
        scores = rng.permutation(np.arange(c, dtype=np.float32) - np.float32(c / 2)).astype(np.float32)
        scores = (scores * np.float32(0.37)).astype(np.float32)
        assert len(np.unique(scores)) == c
        ids = rng.permutation(c).astype(np.int32)
        ob, oi = _oracle_bits(scores[None, :], ids[None, :], k)
        top_t = np.sort(torch.topk(torch.from_numpy(scores), k).indices.numpy())
        top_n = np.sort(np.argpartition(-scores.astype(np.float64), k - 1)[:k]) if k < c else np.arange(c)
        assert np.array_equal(top_t, top_n)
        assert np.array_equal(ob[0], scores[top_t].view(np.uint32))
        assert np.array_equal(oi[0], ids[top_t])


def check_all_tie_rows_pick_lowest_ids(seed=3):
    """Every score equal: the K lowest ids win, emitted in position order."""
    rng = np.random.default_rng(seed)
    for c, k in [(8192, 2048), (300, 7), (64, 64)]:
        ids = rng.permutation(10 * c)[:c].astype(np.int32)
        scores = np.full(c, 2.5, dtype=np.float32)
        ob, oi = _oracle_bits(scores[None], ids[None], k)
        lowest = np.sort(ids)[:k]
        keep = np.isin(ids, lowest)
        assert np.array_equal(oi[0], ids[keep])
        assert np.all(ob[0] == np.float32(2.5).view(np.uint32))


def _check_invariants(scores, ids, k, out_s, out_i):
    """Count, dominance, position order, padding (BJ invariants + readings 3-5)."""
    rows, c = scores.shape
    n_sel = min(k, c)
    bits = scores.view(np.uint32)
    ob = out_s.view(np.uint32)
    for r in range(rows):
        # reconstruct which positions were selected: the output must be an
        # order-preserving subsequence of the row
        sel = np.zeros(c, dtype=bool)
        j = 0
        for p in range(c):
            if j < n_sel and bits[r, p] == ob[r, j] and ids[r, p] == out_i[r, j]:
                sel[p] = True
                j += 1
        assert j == n_sel, f"row {r}: output is not a position-ordered subsequence"
        assert np.all(ob[r, n_sel:] == PAD_BITS) and np.all(out_i[r, n_sel:] == INT32_MAX)
        if n_sel == c:
            continue
        # dominance in the pages' order: worst selected beats best unselected
        sel_c = [(int(bits[r, p]), int(ids[r, p]), p) for p in np.nonzero(sel)[0]]
        uns_c = [(int(bits[r, p]), int(ids[r, p]), p) for p in np.nonzero(~sel)[0]]
        worst = sel_c[0]
        for cnd in sel_c[1:]:
            if _beats(worst, cnd):
                worst = cnd
        best = uns_c[0]
        for cnd in uns_c[1:]:
            if _beats(cnd, best):
                best = cnd
        assert _beats(worst, best), f"row {r}: an unselected candidate beats a selected one"


def check_invariants_on_workloads():
    for g in (W.tiny(), W.tie_heavy(rows=4), W.random_gathered(3, 777, 100, seed=9, dist="special", pad_frac=0.3)):
        out_s, out_i = O.select(g.scores, g.ids, g.k)
        _check_invariants(g.scores, g.ids, g.k, out_s, out_i)


def check_padding_and_short_rows():
    """Empty shards and rows with fewer than K real candidates."""
    c, k = 16, 6
    bits = np.full((3, c), PAD_BITS, dtype=np.uint32)
    ids = np.full((3, c), INT32_MAX, dtype=np.int32)
    # row 1: exactly K real candidates at odd positions, all worse than 0
    real = np.arange(1, 2 * k, 2)
    bits[1, real] = np.float32(-3.0).view(np.uint32)
    ids[1, real] = np.arange(k, dtype=np.int32) + 100
    # row 2: 2 real candidates
    bits[2, [3, 9]] = np.float32(7.0).view(np.uint32)
    ids[2, [3, 9]] = [11, 10]
    ob, oi = _oracle_bits(bits.view(np.float32), ids, k)
    assert np.all(ob[0] == PAD_BITS) and np.all(oi[0] == INT32_MAX)
    assert np.array_equal(oi[1], ids[1, real]) and np.all(ob[1] == np.float32(-3.0).view(np.uint32))
    # both real candidates win; the 4 remaining slots go to the padding
    # candidates with the lowest positions (0, 1, 2, 4), all in position order
    M = INT32_MAX
    assert list(oi[2]) == [M, M, M, 11, M, 10]
    # K larger than the row: everything, then padding
    ob, oi = _oracle_bits(bits[2:3].view(np.float32), ids[2:3], c + 5)
    assert np.array_equal(ob[0, :c], bits[2]) and np.array_equal(oi[0, :c], ids[2])
    assert np.all(ob[0, c:] == PAD_BITS) and np.all(oi[0, c:] == INT32_MAX)


def check_tie_heavy_rows_tie_at_threshold():
    """The tie-heavy workload really ties at the K-th score (the id pass runs)
    and its empty shards never reach the output (brute force on row 0)."""
    g = W.tie_heavy(rows=16)
    out_s, out_i = O.select(g.scores, g.ids, g.k)
    id_pass_rows = 0
    for r in range(g.rows):
        kth = np.sort(g.scores[r])[::-1][g.k - 1]
        above = int(np.sum(g.scores[r] > kth))
        equal = int(np.sum(g.scores[r] == kth))
        assert equal >= 2, "threshold level does not tie"
        id_pass_rows += equal > g.k - above
        assert not np.any(out_i[r] == INT32_MAX)
        # within the tied level the lowest ids win
        tied_ids = np.sort(g.ids[r][g.scores[r] == kth])
        out_tied = np.sort(out_i[r][out_s[r] == kth])
        assert np.array_equal(out_tied, tied_ids[: g.k - above])
    # with seed 4 one row (row 2) fills K exactly at a level boundary, so only
    # 15 of the 16 rows need the id tie-break
    assert id_pass_rows >= g.rows - 2
    # a slice of row 0 across the end of its empty shard (148 padding slots then
    # 152 real candidates): all real ones win, then the first 48 pads by position
    sub = slice(1900, 2200)
    _assert_rows_match_brute(g.scores[0:1, sub].view(np.uint32), g.ids[0:1, sub], 200)


def check_pack_hand_example():
    """Pack (PR #59367, Purpose): id = local index + row start + rank offset;
    a negative local index is an invalid slot -> (-inf, INT32_MAX)."""
    scores = np.array([[0.5, -1.25, 3.0], [2.0, 2.0, -0.0]], dtype=np.float32)
    idx = np.array([[0, 5, -1], [4095, 7, 0]], dtype=np.int32)
    starts = np.array([100, 131071], dtype=np.int32)
    s, i = O.pack(scores, idx, starts, 1000)
    assert i.tolist() == [[1100, 1105, INT32_MAX], [136166, 132078, 132071]]
    sb = s.view(np.uint32)
    assert sb[0, 2] == PAD_BITS
    assert sb[0, 0] == np.float32(0.5).view(np.uint32) and sb[0, 1] == np.float32(-1.25).view(np.uint32)
    assert sb[1, 2] == 0x80000000  # -0.0 copied bit for bit


def check_pack_prefill_properties():
    """On the prefill workload the packed ids of rank r recover the local index
    and stay inside rank r's disjoint range [r*S, r*S + S)."""
    sh = W.prefill(rows=64)
    for r in range(sh.dcp):
        s, i = O.pack(sh.scores[r], sh.local_idx[r], sh.row_starts[r], int(sh.rank_offsets[r]))
        lo = r * W.PREFILL_RANK_STRIDE
        assert np.all((i >= lo) & (i < lo + W.PREFILL_RANK_STRIDE))
        back = i.astype(np.int64) - sh.row_starts[r][:, None] - sh.rank_offsets[r]
        assert np.array_equal(back, sh.local_idx[r])
        assert np.array_equal(s.view(np.uint32), sh.scores[r].view(np.uint32))


def check_merge_hand_example():
    """Two ranks, one row: the gathered row is rank 0's packed slice then rank
    1's, and the merge selects from it (ties -> lowest global id)."""
    sc = np.array([[[1.0, 3.0]], [[3.0, 0.5]]], dtype=np.float32)  # (dcp=2, T=1, Kl=2)
    idx = np.array([[[0, 1]], [[0, 1]]], dtype=np.int32)
    starts = np.array([[10], [10]], dtype=np.int32)
    offs = np.array([0, 100], dtype=np.int32)
    gs, gi = O.gather_rows(sc, idx, starts, offs)
    assert gi.tolist() == [[10, 11, 110, 111]]
    s, i = O.merge(sc, idx, starts, offs, 2)
    assert i.tolist() == [[11, 110]] and s.tolist() == [[3.0, 3.0]]
    s, i = O.merge(sc, idx, starts, offs, 1)
    assert i.tolist() == [[11]]  # 3.0 ties; global id 11 < 110


def check_merge_equals_select_of_gathered():
    """The merge over the prefill workload equals selecting from the gathered
    rows built slice by slice with the rank layout written out here."""
    sh = W.prefill(rows=8, local_k=64)
    c = sh.dcp * sh.local_k
    bits = np.empty((sh.rows, c), np.uint32)
    ids = np.empty((sh.rows, c), np.int32)
    for r in range(sh.dcp):
        bits[:, r * sh.local_k:(r + 1) * sh.local_k] = sh.scores[r].view(np.uint32)
        ids[:, r * sh.local_k:(r + 1) * sh.local_k] = sh.local_idx[r] + sh.row_starts[r][:, None] + sh.rank_offsets[r]
    ms, mi = O.merge(sh.scores, sh.local_idx, sh.row_starts, sh.rank_offsets, 100)
    _assert_rows_match_brute(bits[:2], ids[:2], 100)
    ss, si = O.select(bits.view(np.float32), ids, 100)
    assert np.array_equal(mi, si) and np.array_equal(ms.view(np.uint32), ss.view(np.uint32))


def check_pages_memory_figures():
    """The printed scratch sizes of PR #59367 (Purpose) and the one-GPU share."""
    with open(os.path.join(GOLDEN, "pages_memory_figures.json")) as f:
        fig = json.load(f)
    peak, gather, chunked = fig["cases"]
    v = O.pages_scratch_bytes(peak["rows"], peak["dcp"], peak["local_k"]) / peak["unit_bytes"]
    assert abs(v - peak["value"]) <= peak["rounding"], v
    v = O.gather_output_bytes(gather["rows"], gather["dcp"], gather["local_k"]) / gather["unit_bytes"]
    assert abs(v - gather["value"]) <= gather["rounding"], v
    v = O.pages_scratch_bytes(chunked["rows"], chunked["dcp"], chunked["local_k"]) / chunked["unit_bytes"]
    assert abs(v - chunked["value"]) <= chunked["rounding"], v
    assert O.MERGE_ROWS == fig["merge_rows"]["value"]
    # the one-GPU workspace (one chunk's row-major gathered buffer) stays
    # within the page's chunked bound and does not grow past one chunk
    for rows in (1, 5, 1024, 1025, 8192):
        ws = O.merge_workspace_bytes(rows, 4, 2048)
        assert ws <= O.pages_scratch_bytes(min(rows, 1024), 4, 2048)
        assert ws == O.gather_output_bytes(min(rows, 1024), 4, 2048)


# ----------------------------------------------------------------------------
# local top-K (the step before the merge)
# ----------------------------------------------------------------------------
def _brute_local_row(bits, k, length):
    """Brute-force local top-K of one row: the candidates are the first
    ``length`` columns with id = column; then (-inf, -1) slots."""
    n = len(bits) if length is None else min(max(int(length), 0), len(bits))
    cols = list(range(n))
    eb, ei = brute_select_row([int(b) for b in bits[:n]], cols, k) if n else ([], [])
    m = min(k, n)
    return eb[:m] + [PAD_BITS] * (k - m), ei[:m] + [-1] * (k - m)


def check_local_topk_against_brute(seed=11):
    """Small rows with heavy ties, +-0, +-inf and per-row lengths (including
    0, negative and past the end) against the O(C^2) brute force."""
    rng = np.random.default_rng(seed)
    for dist in ("levels", "special", "normal"):
        for num_cols, k in ((1, 1), (7, 3), (40, 40), (40, 64), (96, 17)):
            d = W.local(rows=5, num_cols=num_cols, k=k, seed=int(rng.integers(1 << 30)), dist=dist)
            lengths = np.array([num_cols, 0, -3, num_cols + 5, num_cols // 2], np.int32)
            for lens in (None, lengths):
                s, i = O.local_topk(d.scores, k, lens)
                sb = np.asarray(s, np.float32).view(np.uint32)
                for t in range(d.rows):
                    eb, ei = _brute_local_row(d.scores[t].view(np.uint32), k, None if lens is None else lens[t])
                    assert [int(x) for x in sb[t]] == eb, (dist, num_cols, k, t)
                    assert [int(x) for x in i[t]] == ei, (dist, num_cols, k, t)


def check_local_topk_distinct_matches_library_topk(seed=12):
    """Distinct scores: the selected columns are torch.topk's, in column order,
    with their scores copied."""
    import torch

    rng = np.random.default_rng(seed)
    # distinct, exactly representable scores (-8 .. 8 in steps of 2^-8)
    scores = np.stack([rng.permutation(4096) for _ in range(8)]).astype(np.float32) / np.float32(256) - np.float32(8)
    s, i = O.local_topk(scores, 2048)
    ref = torch.topk(torch.from_numpy(scores), 2048, dim=1).indices.sort(dim=1).values.numpy()
    assert np.array_equal(i, ref.astype(np.int32))
    assert np.array_equal(s.view(np.uint32), np.take_along_axis(scores, ref, 1).view(np.uint32))


def check_local_topk_all_ties_take_first_columns():
    """A constant row keeps columns 0..k-1; a row of -inf scores too."""
    for value in (1.0, -np.inf):
        scores = np.full((2, 300), value, np.float32)
        s, i = O.local_topk(scores, 120)
        assert np.array_equal(i, np.broadcast_to(np.arange(120, dtype=np.int32), (2, 120)))


def check_local_then_merge_is_global_topk(seed=13):
    """Two stages equal one (PR #47348, Summary: each rank keeps the top-K of
    its shard, the merge takes the global top-K): local top-K per rank with ids
    made global by the pack, then the merge, equals the top-K of the
    concatenated score rows with global ids, written out here column by
    column, in the same position order."""
    rng = np.random.default_rng(seed)
    dcp, rows, cols, k = 4, 6, 96, 40
    for dist in ("levels", "normal"):
        ranks = [W.local(rows=rows, num_cols=cols, k=k, seed=int(rng.integers(1 << 30)), dist=dist)
                 for _ in range(dcp)]
        starts = rng.integers(0, 1000, size=rows, dtype=np.int32)
        offs = np.arange(dcp, dtype=np.int32) * np.int32(1000 + cols)
        loc = [O.local_topk(d.scores, k) for d in ranks]
        ms, mi = O.merge(np.stack([l[0] for l in loc]), np.stack([l[1] for l in loc]),
                         np.stack([starts] * dcp), offs, k)
        bits = np.concatenate([d.scores.view(np.uint32) for d in ranks], axis=1)
        gid = np.empty((rows, dcp * cols), np.int32)
        for r in range(dcp):
            for c in range(cols):
                gid[:, r * cols + c] = c + starts + offs[r]
        for t in range(rows):
            eb, ei = brute_select_row(bits[t], gid[t], k)
            assert [int(x) for x in ms[t].view(np.uint32)] == eb, (dist, t)
            assert [int(x) for x in mi[t]] == ei, (dist, t)


ALL_CHECKS = [
    check_score_key_ladder,
    check_score_key_orders_like_floats,
    check_exhaustive_tiny_rows,
    check_random_rows_with_specials,
    check_configs_tiny_against_brute,
    check_distinct_scores_match_library_topk,
    check_all_tie_rows_pick_lowest_ids,
    check_invariants_on_workloads,
    check_padding_and_short_rows,
    check_tie_heavy_rows_tie_at_threshold,
    check_pack_hand_example,
    check_pack_prefill_properties,
    check_merge_hand_example,
    check_merge_equals_select_of_gathered,
    check_pages_memory_figures,
    check_local_topk_against_brute,
    check_local_topk_distinct_matches_library_topk,
    check_local_topk_all_ties_take_first_columns,
    check_local_then_merge_is_global_topk,
]
