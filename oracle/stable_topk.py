"""CPU oracle: stable global top-K over gathered DCP candidates, pack, chunked merge.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call this module.  The HIP library never calls it, and this module
shares no code, table or helper with the HIP library; both sides take their
inputs from ``stable_top_selection_amd.workloads`` only.

Sources (vLLM pull-request pages):

* PR #47348, "[Kernel] Optimize CuTeDSL DCP top-k merge", Summary, commit 1:
  the merge picks each row's global top-K among the gathered candidates, by
  score descending and, among equal scores, by the lowest global token id; the
  selection is deterministic.  The selector it replaced always sorted a 64-bit
  key whose high word is the 32-bit score key and whose low word is the bitwise
  complement of the token id; the new selector works on 32-bit score keys first.
* PR #50009, "[DCP][Performance] Add Shared-DCP peer-addressable decode data
  paths", Top-K performance: the stable top-K consumer can load every owner's
  candidate shard in place rather than from a gathered copy (the fused merge
  computes the same result as ``merge``); each rank keeps 2048 candidates out
  of 4096 local score columns (the local top-K step, ``local_topk``).
* PR #59367, "[Bugfix][Attention] Reserve the sparse indexer's DCP top-k merge
  scratch through the workspace manager", Purpose: the pack step turns each
  rank's local top-K into packed (score, global id) candidates using a per-row
  row start; the gathered buffer the selector reads is row-major with the rank
  dimension inside the row; the merge walks the rows 1024 at a time and, the
  selector being row-independent, the result does not change; the scratch of the
  unchunked merge is (1 + 2 dcp) * 8 * T * K bytes per rank.

Readings where the pages leave a step open (each is pinned by a test, see
``tests/test_oracle_pins.py``):

1. Score key: the standard order-preserving map of fp32 bits to uint32 (flip
   every bit of a negative float, set the sign bit of a non-negative one).  It
   orders -0 below +0, +NaN above +inf and -NaN below -inf (IEEE 754 totalOrder).
2. Ids compare as uint32 through their bitwise complement, as in the 64-bit key;
   for non-negative ids this is "lowest id first".
3. Candidates with the same score bits and the same id: the lower position in
   the gathered row wins (a stable sort).
4. Output order: the selected candidates are written in candidate-position
   order, (score bits, id) copied unchanged.
5. K larger than the row: every candidate is selected and slots [C, K) hold the
   padding candidate (-inf, INT32_MAX).
6. Pack: global id = local index + row start + rank offset, wrapped to int32;
   a negative local index marks an invalid slot and packs to (-inf, INT32_MAX).
7. Local top-K (its tie rule is not on the pages): the merge's order with the
   column as the id, so equal scores go to the lowest column; the selected
   columns are written in column order; a row with fewer valid columns than k
   (per-row lengths) is followed by (-inf, -1) slots, the invalid local slot
   that the pack step recognises.
"""
from __future__ import annotations

import numpy as np

INT32_MAX = 2**31 - 1
PAD_SCORE_BITS = np.uint32(0xFF800000)  # fp32 -inf
PAD_ID = np.int32(INT32_MAX)
MERGE_ROWS = 1024  # rows per chunk of the merge (PR #59367, Purpose)
CANDIDATE_BYTES = 8  # fp32 score + int32 id (PR #59367, Purpose: packed (T, K, 2) fp32)


def score_key(scores: np.ndarray) -> np.ndarray:
    """uint32 key that orders like the fp32 scores (reading 1).

    PR #47348, Summary, commit 1: the radix pass runs over 32-bit score keys.
    """
    b = np.ascontiguousarray(scores, dtype=np.float32).view(np.uint32)
    negative = (b >> np.uint32(31)) == 1
    return np.where(negative, ~b, b | np.uint32(0x80000000)).astype(np.uint32)


def sort_key64(scores: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """The 64-bit key of the selector that always sorted: score key in the high
    word, complement of the id in the low word (PR #47348, Summary, commit 1;
    also the bit-exact reference of the heavy-tie trials in the review comment
    on that page).  Larger key = better candidate."""
    hi = score_key(scores).astype(np.uint64) << np.uint64(32)
    lo = (~np.ascontiguousarray(ids, dtype=np.int32).view(np.uint32)).astype(np.uint64)
    return hi | lo


def select(scores: np.ndarray, ids: np.ndarray, k: int, row_block: int = 256):
    """Stable global top-K of each row of a gathered candidate buffer.

    ``scores`` float32 (rows, C), ``ids`` int32 (rows, C).  Returns
    (out_scores float32 (rows, k), out_ids int32 (rows, k)).

    Definition (PR #47348, Summary): order the row's candidates by the 64-bit
    key, largest first, and among equal keys by position (reading 3); keep the
    first min(k, C); write them back in position order (reading 4); pad the
    rest (reading 5).
    """
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    if scores.shape != ids.shape or scores.ndim != 2:
        raise ValueError("scores and ids must both be (rows, C)")
    if k < 1:
        raise ValueError("k must be >= 1")
    rows, c = scores.shape
    n_sel = min(k, c)
    out_bits = np.full((rows, k), PAD_SCORE_BITS, dtype=np.uint32)
    out_ids = np.full((rows, k), PAD_ID, dtype=np.int32)
    score_bits = scores.view(np.uint32)
    for r0 in range(0, rows, row_block):
        r1 = min(rows, r0 + row_block)
        key = sort_key64(scores[r0:r1], ids[r0:r1])
        # ~key reverses the order of uint64, and a stable ascending sort keeps
        # equal keys in position order: largest key first, lowest position first.
        order = np.argsort(~key, axis=1, kind="stable")
        chosen = np.sort(order[:, :n_sel], axis=1)
        out_bits[r0:r1, :n_sel] = np.take_along_axis(score_bits[r0:r1], chosen, axis=1)
        out_ids[r0:r1, :n_sel] = np.take_along_axis(ids[r0:r1], chosen, axis=1)
    return out_bits.view(np.float32), out_ids


LOCAL_PAD_INDEX = np.int32(-1)


def local_topk(scores: np.ndarray, k: int, lengths: np.ndarray | None = None):
    """One rank's local top-K of its indexer scores (reading 7).

    PR #47348, Summary: every DCP rank holds the local top-K of its shard;
    PR #50009, Top-K performance: 2048 of 4096 local score columns.
    ``scores`` float32 (rows, num_cols); ``lengths`` int32 (rows,) or None
    (row t's candidates are its first clamp(lengths[t], 0, num_cols) columns).
    Returns (out_scores float32 (rows, k), out_idx int32 (rows, k)).

    Per row: order the valid columns by score key, largest first, and among
    equal keys by column, lowest first; keep the first min(k, len); write them
    in column order; fill the remaining slots with (-inf, -1).
    """
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    if scores.ndim != 2:
        raise ValueError("scores must be (rows, num_cols)")
    if k < 1:
        raise ValueError("k must be >= 1")
    rows, num_cols = scores.shape
    out_bits = np.full((rows, k), PAD_SCORE_BITS, dtype=np.uint32)
    out_idx = np.full((rows, k), LOCAL_PAD_INDEX, dtype=np.int32)
    bits = scores.view(np.uint32)
    for t in range(rows):
        n = num_cols if lengths is None else int(min(max(int(lengths[t]), 0), num_cols))
        key = score_key(scores[t, :n])
        # ascending stable sort of the complemented key: largest key first,
        # equal keys in column order
        order = np.argsort(~key, kind="stable")
        chosen = np.sort(order[:min(k, n)])
        out_bits[t, :chosen.size] = bits[t, chosen]
        out_idx[t, :chosen.size] = chosen.astype(np.int32)
    return out_bits.view(np.float32), out_idx


def pack(local_scores: np.ndarray, local_idx: np.ndarray, row_starts: np.ndarray, rank_offset: int):
    """One rank's local top-K -> packed (score, global id) candidates (reading 6).

    PR #59367, Purpose: the pack kernel takes a row start per row.
    ``local_scores`` float32 (T, local_k), ``local_idx`` int32 (T, local_k),
    ``row_starts`` int32 (T,).  Returns (scores float32, ids int32), (T, local_k).
    """
    local_idx = np.asarray(local_idx, dtype=np.int32)
    gid = local_idx.astype(np.int64) + np.asarray(row_starts, np.int64)[:, None] + np.int64(rank_offset)
    gid32 = (gid & np.int64(0xFFFFFFFF)).astype(np.uint32).view(np.int32)
    invalid = local_idx < 0
    bits = np.where(invalid, PAD_SCORE_BITS, np.ascontiguousarray(local_scores, np.float32).view(np.uint32))
    ids = np.where(invalid, PAD_ID, gid32).astype(np.int32)
    return bits.astype(np.uint32).view(np.float32), ids


def gather_rows(local_scores, local_idx, row_starts, rank_offsets):
    """Row-major gathered buffer of the merge: rank r's packed candidates of row
    t at columns [r*local_k, (r+1)*local_k) (PR #59367, Purpose: the rank
    dimension is moved inside the row before the selector reads it).

    Inputs are (dcp, T, local_k), (dcp, T, local_k), (dcp, T), (dcp,).
    """
    dcp = len(local_scores)
    parts = [pack(local_scores[r], local_idx[r], row_starts[r], int(rank_offsets[r])) for r in range(dcp)]
    scores = np.concatenate([p[0] for p in parts], axis=1)
    ids = np.concatenate([p[1] for p in parts], axis=1)
    return scores, ids


def merge(local_scores, local_idx, row_starts, rank_offsets, k: int):
    """Global top-K of the DCP merge: pack every rank, gather row-major, select.

    The chunked driver walks the rows 1024 at a time; the selector is
    row-independent, so its result equals this chunk-free definition
    (PR #59367, Purpose).
    """
    scores, ids = gather_rows(local_scores, local_idx, row_starts, rank_offsets)
    return select(scores, ids, k)


def pages_scratch_bytes(rows: int, dcp: int, local_k: int) -> int:
    """Peak scratch of the merge on one rank as PR #59367 (Purpose) counts it:
    the packed candidates, the rank-major all-gather output and the copy that
    moves the rank dimension, (1 + 2 dcp) * 8 * rows * K bytes."""
    return (1 + 2 * dcp) * CANDIDATE_BYTES * rows * local_k


def gather_output_bytes(rows: int, dcp: int, local_k: int) -> int:
    """Size of the all-gather output (dcp * rows, K, 2) fp32 (PR #59367, Purpose)."""
    return dcp * rows * local_k * CANDIDATE_BYTES


def merge_workspace_bytes(rows: int, dcp: int, local_k: int) -> int:
    """Workspace of the one-GPU chunked merge: one chunk's row-major gathered
    buffer, min(rows, 1024) * dcp * local_k candidates of 8 bytes.  Nothing is
    exchanged on one GPU, so the packed and rank-major buffers that the pages
    count are not needed; the pack step writes straight into this buffer."""
    return min(rows, MERGE_ROWS) * dcp * local_k * CANDIDATE_BYTES
