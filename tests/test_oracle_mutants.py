"""Plant plausible mistakes in the CPU oracle and check that its pins catch them.

Each mutant replaces one oracle function (on the CPU, through monkeypatch) with
a version that has one mistake; the test passes only if at least one check of
``oracle_checks.ALL_CHECKS`` then fails.  This shows the pins are strong enough
that a dropped term, a wrong sign, a wrong index or a wrong order would not go
unnoticed.
"""
import numpy as np
import pytest

import oracle_checks as C
from oracle import stable_topk as O

_ORIG_SCORE_KEY = O.score_key
_ORIG_PACK = O.pack
_ORIG_LOCAL = O.local_topk


def _key_no_negative_flip(scores):
    b = np.ascontiguousarray(scores, dtype=np.float32).view(np.uint32)
    return (b | np.uint32(0x80000000)).astype(np.uint32)


def _key_sign_xor_only(scores):
    b = np.ascontiguousarray(scores, dtype=np.float32).view(np.uint32)
    return (b ^ np.uint32(0x80000000)).astype(np.uint32)


def _key_truncated(scores):
    k = _ORIG_SCORE_KEY(scores)
    return (k >> np.uint32(4)) << np.uint32(4)


def _key_zero_canonical(scores):
    # -0 given the key of +0, as a float comparison would treat them
    s = np.ascontiguousarray(scores, dtype=np.float32)
    return _ORIG_SCORE_KEY(np.where(s == 0, np.float32(0.0), s))


def _key_nan_top(scores):
    # every NaN, whatever its sign, ordered above +inf
    s = np.ascontiguousarray(scores, dtype=np.float32)
    return np.where(np.isnan(s), np.uint32(0xFFFFFFFF), _ORIG_SCORE_KEY(s)).astype(np.uint32)


def _key64_plain_id(scores, ids):
    hi = O.score_key(scores).astype(np.uint64) << np.uint64(32)
    return hi | np.ascontiguousarray(ids, np.int32).view(np.uint32).astype(np.uint64)


def _make_select(mistake):
    def select(scores, ids, k, row_block=256):
        scores = np.ascontiguousarray(scores, dtype=np.float32)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        rows, c = scores.shape
        n_sel = min(k, c)
        if mistake == "off_by_one" and 1 < n_sel < c:
            n_sel -= 1
        pad_bits = np.uint32(0) if mistake == "pad_zero" else np.uint32(0xFF800000)
        out_bits = np.full((rows, k), pad_bits, dtype=np.uint32)
        out_ids = np.full((rows, k), np.int32(-1) if mistake == "pad_id_minus_one" else np.int32(2**31 - 1),
                          dtype=np.int32)
        key = O.sort_key64(scores, ids)
        if mistake == "last_position_wins":
            order = np.argsort(key, axis=1, kind="stable")[:, ::-1]
        else:
            order = np.argsort(~key, axis=1, kind="stable")
        chosen = order[:, :n_sel]
        if mistake != "score_order_output":
            chosen = np.sort(chosen, axis=1)
        out_bits[:, :n_sel] = np.take_along_axis(scores.view(np.uint32), chosen, axis=1)
        out_ids[:, :n_sel] = np.take_along_axis(ids, chosen, axis=1)
        return out_bits.view(np.float32), out_ids

    return select


def _make_pack(mistake):
    orig = _ORIG_PACK

    def pack(local_scores, local_idx, row_starts, rank_offset):
        if mistake == "no_rank_offset":
            return orig(local_scores, local_idx, row_starts, 0)
        if mistake == "invalid_keeps_score":
            s, i = orig(local_scores, local_idx, row_starts, rank_offset)
            s = np.where(np.asarray(local_idx) < 0, np.asarray(local_scores, np.float32), s).astype(np.float32)
            return s, i
        if mistake == "row_start_of_next_row":
            rs = np.roll(np.asarray(row_starts), -1)
            return orig(local_scores, local_idx, rs, rank_offset)
        raise AssertionError(mistake)

    return pack


def _gather_reversed(local_scores, local_idx, row_starts, rank_offsets):
    dcp = len(local_scores)
    parts = [O.pack(local_scores[r], local_idx[r], row_starts[r], int(rank_offsets[r])) for r in range(dcp)][::-1]
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1)


def _make_local(mistake):
    def local_topk(scores, k, lengths=None):
        scores = np.ascontiguousarray(scores, dtype=np.float32)
        rows, num_cols = scores.shape
        if mistake == "ignores_lengths":
            return _ORIG_LOCAL(scores, k, None)
        out_bits = np.full((rows, k), np.uint32(0xFF800000), dtype=np.uint32)
        out_idx = np.full((rows, k), np.int32(2**31 - 1) if mistake == "pad_intmax" else np.int32(-1), np.int32)
        for t in range(rows):
            n = num_cols if lengths is None else int(min(max(int(lengths[t]), 0), num_cols))
            if mistake == "lengths_off_by_one" and lengths is not None:
                n = int(min(max(int(lengths[t]) - 1, 0), num_cols))
            key = O.score_key(scores[t, :n])
            if mistake == "ties_highest_column":
                order = np.argsort(key, kind="stable")[::-1]
            else:
                order = np.argsort(~key, kind="stable")
            chosen = order[:min(k, n)]
            if mistake != "score_order_output":
                chosen = np.sort(chosen)
            out_bits[t, :chosen.size] = scores[t].view(np.uint32)[chosen]
            out_idx[t, :chosen.size] = chosen
        return out_bits.view(np.float32), out_idx

    return local_topk


MUTANTS = {
    "key_no_negative_flip": ("score_key", _key_no_negative_flip),
    "key_sign_xor_only": ("score_key", _key_sign_xor_only),
    "key_truncated_low_bits": ("score_key", _key_truncated),
    "key_zero_canonical": ("score_key", _key_zero_canonical),
    "key_nan_top": ("score_key", _key_nan_top),
    "key64_plain_id": ("sort_key64", _key64_plain_id),
    "select_last_position_wins": ("select", _make_select("last_position_wins")),
    "select_score_order_output": ("select", _make_select("score_order_output")),
    "select_pad_zero": ("select", _make_select("pad_zero")),
    "select_off_by_one": ("select", _make_select("off_by_one")),
    "select_pad_id_minus_one": ("select", _make_select("pad_id_minus_one")),
    "pack_no_rank_offset": ("pack", _make_pack("no_rank_offset")),
    "pack_invalid_keeps_score": ("pack", _make_pack("invalid_keeps_score")),
    "pack_wrong_row_start": ("pack", _make_pack("row_start_of_next_row")),
    "gather_ranks_reversed": ("gather_rows", _gather_reversed),
    "scratch_one_dcp_term": ("pages_scratch_bytes", lambda rows, dcp, k: (1 + dcp) * 8 * rows * k),
    "workspace_not_chunked": ("merge_workspace_bytes", lambda rows, dcp, k: rows * dcp * k * 8),
    "local_ties_highest_column": ("local_topk", _make_local("ties_highest_column")),
    "local_score_order_output": ("local_topk", _make_local("score_order_output")),
    "local_pad_intmax": ("local_topk", _make_local("pad_intmax")),
    "local_ignores_lengths": ("local_topk", _make_local("ignores_lengths")),
    "local_lengths_off_by_one": ("local_topk", _make_local("lengths_off_by_one")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for check in C.ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError) as e:  # a failing pin
            caught.append(f"{check.__name__}: {type(e).__name__}")
            break
    assert caught, f"mutant {name} survived every pin"
