"""Seeded synthetic inputs for the DCP top-K merge.

This module only draws random numbers and lays them out; it holds none of the
selection, packing or key arithmetic.  Both the CPU oracle tests and the HIP
parity tests take their inputs from here, so the two sides always see the same
bits.

Workload shapes follow the merge described on vLLM PR #47348 ("Optimize
CuTeDSL DCP top-k merge", Summary and Benchmarks) and vLLM PR #59367 ("Reserve
the sparse indexer's DCP top-k merge scratch through the workspace manager",
Purpose): every DCP rank contributes its local top-K candidates of one query row,
each candidate is an (fp32 score, int32 global token id) pair, and the gathered
row holds rank r's candidates at columns [r*local_k, (r+1)*local_k).

Recipes (numpy PCG64, ``np.random.default_rng(seed)``):

* ``tiny``       4 rows, DCP 4 x local K 64 = 256 candidates, K 64, scores
                 N(0,1); rank r ids are 64 distinct ints from [r*1024, (r+1)*1024).
* ``decode``     rows 16 (also 1/8/32/64), DCP 4 x 2048 = 8192 candidates, K 2048,
                 scores N(0,1); rank r ids distinct from [r*32768, (r+1)*32768).
* ``large``      256 rows x 8192 candidates, K 2048, scores U(-10,10); rank r ids
                 distinct from [r*65536, (r+1)*65536).
* ``tie_heavy``  16 rows x 8192, K 2048, scores from 16 exact levels
                 {-7.5, -6.5, ..., 7.5}; in rows with row % 4 == 0, rank
                 (row // 4) % 4 is an empty shard: all its slots hold the padding
                 candidate (-inf, INT32_MAX).
* ``prefill``    T rows (8192 at full size), DCP 4, local K 2048, K 2048: per rank
                 fp32 scores N(0,1), local indices distinct per row from [0, 4096),
                 per-row row starts U[0, 131072) shared by the ranks, and rank
                 offsets r * 135168 (131072 + 4096, the smallest stride that keeps
                 the ranks' id ranges disjoint).

* ``fused``      the prefill recipe at 256 rows (seed 7): the per-rank arrays
                 that the fused merge reads in place, the same shape as
                 ``large`` (8192 candidates per row, K 2048).
* ``local``      one rank's indexer scores before its local top-K: rows 64 (also
                 1/8/32 and 256), 4096 columns, k 2048 (vLLM PR #50009, "Add
                 Shared-DCP peer-addressable decode data paths", Top-K
                 performance: 2048 candidates per rank out of 4096 local score
                 columns), scores N(0,1); optional per-row lengths U[0, 4096].

Within a rank's slice, candidates appear in generation order (neither scores nor
ids are sorted).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

INT32_MAX = np.int32(2**31 - 1)
PAD_SCORE = np.float32(-np.inf)
PREFILL_ROW_START_SPAN = 131072
PREFILL_LOCAL_COLUMNS = 4096
PREFILL_RANK_STRIDE = PREFILL_ROW_START_SPAN + PREFILL_LOCAL_COLUMNS


@dataclass
class Gathered:
    """A row-major gathered candidate buffer: ``scores``/``ids`` are (rows, C)."""

    name: str
    scores: np.ndarray  # float32 (rows, C)
    ids: np.ndarray  # int32 (rows, C)
    k: int
    dcp: int = 1
    local_k: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return int(self.scores.shape[0])

    @property
    def num_cand(self) -> int:
        return int(self.scores.shape[1])

    def interleaved(self) -> np.ndarray:
        """(rows, C, 2) int32 words: [..., 0] = score bits, [..., 1] = id."""
        out = np.empty(self.scores.shape + (2,), dtype=np.int32)
        out[..., 0] = self.scores.view(np.int32)
        out[..., 1] = self.ids
        return out

    def digest(self) -> str:
        h = hashlib.sha256()
        h.update(np.ascontiguousarray(self.scores).view(np.uint8))
        h.update(np.ascontiguousarray(self.ids).view(np.uint8))
        return h.hexdigest()[:16]


@dataclass
class LocalShards:
    """Per-rank local top-K outputs before packing.

    ``scores`` and ``local_idx`` are (dcp, T, local_k); ``row_starts`` is
    (dcp, T); ``rank_offsets`` is (dcp,).
    """

    name: str
    scores: np.ndarray
    local_idx: np.ndarray
    row_starts: np.ndarray
    rank_offsets: np.ndarray
    k: int

    @property
    def dcp(self) -> int:
        return int(self.scores.shape[0])

    @property
    def rows(self) -> int:
        return int(self.scores.shape[1])

    @property
    def local_k(self) -> int:
        return int(self.scores.shape[2])

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in (self.scores, self.local_idx, self.row_starts, self.rank_offsets):
            h.update(np.ascontiguousarray(a).view(np.uint8))
        return h.hexdigest()[:16]


@dataclass
class DenseScores:
    """One rank's indexer scores: ``scores`` (rows, num_cols) float32 and, if
    not None, ``lengths`` (rows,) int32 valid columns per row."""

    name: str
    scores: np.ndarray
    k: int
    lengths: np.ndarray | None = None

    @property
    def rows(self) -> int:
        return int(self.scores.shape[0])

    @property
    def num_cols(self) -> int:
        return int(self.scores.shape[1])


def distinct_per_row(rng: np.random.Generator, rows: int, count: int, span: int) -> np.ndarray:
    """(rows, count) int32: each row holds ``count`` distinct ints from [0, span)."""
    if count > span:
        raise ValueError("count exceeds span")
    base = np.broadcast_to(np.arange(span, dtype=np.int32), (rows, span)).copy()
    return np.ascontiguousarray(rng.permuted(base, axis=1)[:, :count])


def _rank_ids(rng, rows, dcp, local_k, span):
    """Ids for a gathered row: rank r's slice is distinct within [r*span, (r+1)*span)."""
    ids = np.empty((rows, dcp * local_k), dtype=np.int32)
    for r in range(dcp):
        ids[:, r * local_k:(r + 1) * local_k] = distinct_per_row(rng, rows, local_k, span) + np.int32(r * span)
    return ids


def tiny(seed: int = 1) -> Gathered:
    rng = np.random.default_rng(seed)
    rows, dcp, local_k = 4, 4, 64
    scores = rng.standard_normal((rows, dcp * local_k), dtype=np.float32)
    ids = _rank_ids(rng, rows, dcp, local_k, 1024)
    return Gathered("tiny", scores, ids, k=64, dcp=dcp, local_k=local_k)


def decode(rows: int = 16, seed: int | None = None) -> Gathered:
    rng = np.random.default_rng([2, rows] if seed is None else seed)
    dcp, local_k = 4, 2048
    scores = rng.standard_normal((rows, dcp * local_k), dtype=np.float32)
    ids = _rank_ids(rng, rows, dcp, local_k, 32768)
    return Gathered(f"decode_rows{rows}", scores, ids, k=2048, dcp=dcp, local_k=local_k)


def large(rows: int = 256, seed: int = 3) -> Gathered:
    rng = np.random.default_rng(seed)
    dcp, local_k = 4, 2048
    scores = (rng.random((rows, dcp * local_k), dtype=np.float32) * np.float32(20.0) - np.float32(10.0)).astype(np.float32)
    ids = _rank_ids(rng, rows, dcp, local_k, 65536)
    return Gathered(f"large_rows{rows}", scores, ids, k=2048, dcp=dcp, local_k=local_k)


TIE_LEVELS = (np.arange(16, dtype=np.float32) - np.float32(7.5)).astype(np.float32)


def tie_heavy(rows: int = 16, seed: int = 4) -> Gathered:
    rng = np.random.default_rng(seed)
    dcp, local_k = 4, 2048
    scores = TIE_LEVELS[rng.integers(0, 16, size=(rows, dcp * local_k))]
    ids = _rank_ids(rng, rows, dcp, local_k, 32768)
    empty = []
    for row in range(0, rows, 4):
        r = (row // 4) % dcp
        scores[row, r * local_k:(r + 1) * local_k] = PAD_SCORE
        ids[row, r * local_k:(r + 1) * local_k] = INT32_MAX
        empty.append((row, r))
    return Gathered(f"tie_heavy_rows{rows}", np.ascontiguousarray(scores), ids, k=2048, dcp=dcp,
                    local_k=local_k, meta={"empty_shards": empty})


def short_context(rows: int = 16, seed: int = 8, min_len: int = 64) -> Gathered:
    """A decode batch whose contexts are shorter than K: row r's context of
    L_r ~ U[min_len, 2048) tokens is spread over the 4 ranks token by token,
    so rank j holds ceil((L_r - j) / 4) valid entries at the start of its
    2048-slot slice and padding after them.  Every real candidate is selected
    and the threshold falls among the padding."""
    rng = np.random.default_rng(seed)
    dcp, local_k = 4, 2048
    scores = rng.standard_normal((rows, dcp * local_k), dtype=np.float32)
    ids = _rank_ids(rng, rows, dcp, local_k, 32768)
    lengths = rng.integers(min_len, local_k, size=rows)
    for row, length in enumerate(lengths):
        for r in range(dcp):
            valid = max(0, -(-(int(length) - r) // dcp))
            scores[row, r * local_k + valid:(r + 1) * local_k] = PAD_SCORE
            ids[row, r * local_k + valid:(r + 1) * local_k] = INT32_MAX
    return Gathered(f"short_context_rows{rows}", np.ascontiguousarray(scores), ids, k=2048, dcp=dcp,
                    local_k=local_k, meta={"context_lengths": [int(x) for x in lengths]})


def prefill(rows: int = 8192, seed: int = 5, dcp: int = 4, local_k: int = 2048,
            invalid_frac: float = 0.0) -> LocalShards:
    """``invalid_frac`` of the local slots, chosen at random after the draws
    above, get local index -1 (an invalid slot)."""
    rng = np.random.default_rng(seed)
    scores = rng.standard_normal((dcp, rows, local_k), dtype=np.float32)
    local_idx = np.empty((dcp, rows, local_k), dtype=np.int32)
    for r in range(dcp):
        local_idx[r] = distinct_per_row(rng, rows, local_k, max(PREFILL_LOCAL_COLUMNS, local_k))
    starts = rng.integers(0, PREFILL_ROW_START_SPAN, size=rows, dtype=np.int32)
    row_starts = np.ascontiguousarray(np.broadcast_to(starts, (dcp, rows)))
    rank_offsets = (np.arange(dcp, dtype=np.int32) * np.int32(PREFILL_RANK_STRIDE)).astype(np.int32)
    if invalid_frac > 0.0:
        local_idx = np.where(rng.random(local_idx.shape) < invalid_frac, np.int32(-1), local_idx).astype(np.int32)
    return LocalShards(f"prefill_T{rows}", scores, local_idx, row_starts, rank_offsets, k=2048)


def fused(rows: int = 256, seed: int = 7) -> LocalShards:
    sh = prefill(rows=rows, seed=seed)
    sh.name = f"fused_rows{rows}"
    return sh


def local(rows: int = 64, num_cols: int = 4096, k: int = 2048, seed: int | None = None,
          dist: str = "normal", with_lengths: bool = False) -> DenseScores:
    """``dist``: ``normal`` (N(0,1)), ``levels`` (the 16 tie levels) or
    ``special`` (the +-0 / +-inf / finite mix of ``random_gathered``)."""
    rng = np.random.default_rng([6, rows, num_cols, k] if seed is None else seed)
    shape = (rows, num_cols)
    if dist == "normal":
        scores = rng.standard_normal(shape, dtype=np.float32)
    elif dist == "levels":
        scores = TIE_LEVELS[rng.integers(0, 16, size=shape)]
    elif dist == "special":
        alphabet = np.array([-np.inf, -2.0, -1.0, -0.0, 0.0, 1.0, 2.0, np.inf], dtype=np.float32)
        scores = alphabet[rng.integers(0, alphabet.size, size=shape)]
    else:
        raise ValueError(dist)
    lengths = rng.integers(0, num_cols + 1, size=rows, dtype=np.int32) if with_lengths else None
    return DenseScores(f"local_{dist}_{rows}x{num_cols}_k{k}", np.ascontiguousarray(scores), k=k, lengths=lengths)


def random_gathered(rows: int, num_cand: int, k: int, seed: int, dist: str = "normal",
                    id_span: int | None = None, pad_frac: float = 0.0,
                    repeat_ids: bool = False) -> Gathered:
    """Ragged-size parity inputs: ids distinct per row from [0, id_span).

    With ``repeat_ids`` the ids are drawn with replacement from [0, id_span), so
    a row can hold several candidates with the same (score, id) pair.

    ``dist`` is ``normal`` (N(0,1)), ``uniform`` (U(-10,10)), ``levels`` (the 16
    tie levels), ``const`` (every score 1.0) or ``special`` (a mix that includes
    +-0, +-inf and finite values).  ``pad_frac`` of the slots, chosen at random,
    become padding candidates.
    """
    rng = np.random.default_rng(seed)
    shape = (rows, num_cand)
    if dist == "normal":
        scores = rng.standard_normal(shape, dtype=np.float32)
    elif dist == "uniform":
        scores = (rng.random(shape, dtype=np.float32) * np.float32(20.0) - np.float32(10.0)).astype(np.float32)
    elif dist == "levels":
        scores = TIE_LEVELS[rng.integers(0, 16, size=shape)]
    elif dist == "const":
        scores = np.ones(shape, dtype=np.float32)
    elif dist == "special":
        alphabet = np.array([-np.inf, -2.0, -1.0, -0.0, 0.0, 1.0, 2.0, np.inf], dtype=np.float32)
        scores = alphabet[rng.integers(0, alphabet.size, size=shape)]
    else:
        raise ValueError(dist)
    span = id_span if id_span is not None else max(4 * num_cand, 1)
    if repeat_ids:
        ids = rng.integers(0, span, size=shape, dtype=np.int32)
    elif num_cand:
        ids = distinct_per_row(rng, rows, num_cand, span)
    else:
        ids = np.zeros(shape, np.int32)
    if pad_frac > 0.0:
        mask = rng.random(shape) < pad_frac
        scores = np.where(mask, PAD_SCORE, scores).astype(np.float32)
        ids = np.where(mask, INT32_MAX, ids).astype(np.int32)
    return Gathered(f"random_{dist}_{rows}x{num_cand}_k{k}_s{seed}", np.ascontiguousarray(scores),
                    np.ascontiguousarray(ids), k=k)


def block_heads(rows: int, seed: int, heads_high: bool, num_cand: int = 8192, k: int = 2048) -> Gathered:
    """Rows whose first 256 candidates of every 1024-candidate block come from
    another distribution than the rest: N(0,1) heads and N(6,1) tails, or the
    reverse (``heads_high``).  Ids distinct per row."""
    rng = np.random.default_rng(seed)
    head = (np.arange(num_cand) % 1024) < 256
    lo = rng.standard_normal((rows, num_cand), dtype=np.float32)
    hi = (rng.standard_normal((rows, num_cand), dtype=np.float32) + np.float32(6.0)).astype(np.float32)
    scores = np.where(head, hi, lo) if heads_high else np.where(head, lo, hi)
    ids = distinct_per_row(rng, rows, num_cand, 4 * num_cand)
    return Gathered(f"block_heads_{'high' if heads_high else 'low'}_{rows}x{num_cand}_k{k}",
                    np.ascontiguousarray(scores.astype(np.float32)), ids, k=k)


def crowded(rows: int, seed: int, tie: bool, num_cand: int = 8192, k: int = 2048) -> Gathered:
    """Rows with a crowd of 64 near-equal scores (5.45 + 1e-6 N(0,1), or
    exactly 5.45 with ``tie``) inside 1000 scores U(5.0, 5.9), above them 1500
    scores U(10, 20), below them the rest U(-20, -10); positions shuffled.
    With k = 2048 the k-th best score falls among the crowd."""
    rng = np.random.default_rng(seed)
    n_top, n_mid, n_crowd = 1500, 1000, 64
    n_low = num_cand - n_top - n_mid - n_crowd
    scores = np.empty((rows, num_cand), dtype=np.float32)
    for r in range(rows):
        crowd = np.full(n_crowd, 5.45, dtype=np.float32) if tie else \
            (np.float32(5.45) + np.float32(1e-6) * rng.standard_normal(n_crowd, dtype=np.float32)).astype(np.float32)
        parts = [rng.uniform(10.0, 20.0, n_top), rng.uniform(5.0, 5.9, n_mid), crowd,
                 rng.uniform(-20.0, -10.0, n_low)]
        row = np.concatenate([x.astype(np.float32) for x in parts])
        scores[r] = row[rng.permutation(num_cand)]
    ids = distinct_per_row(rng, rows, num_cand, 4 * num_cand)
    return Gathered(f"crowded_{'tie' if tie else 'distinct'}_{rows}x{num_cand}_k{k}", scores, ids, k=k)


CONFIG_NAMES = ("tiny", "decode", "large", "tie_heavy", "prefill")
