"""Seeded random shapes through every selecting entry point, bit for bit
against the oracle.

The other GPU tests pick their shapes by hand (tile boundaries, the pages'
workloads, degenerate rows).  Here fixed seeds draw about a thousand more:
candidate counts log-uniform over [1, 16384], k below, near and above the
count, five score distributions with optional padding and repeated ids,
misaligned buffers, the split-row path at 1 to 8 parts, the local top-K with
and without per-row lengths, and the fused merge over 1 to 16 ranks.  Each
case prints its parameters before it runs.  DCPTOPK_FUZZ_SCALE=n runs n times
as many blocks of cases (the first blocks are always the default run's).
"""
import os

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, gpu_select, to_dev
from oracle import stable_topk as O
from stable_top_selection_amd import binding as B
from stable_top_selection_amd import workloads as W

pytestmark = pytest.mark.gpu

DISTS = ["normal", "uniform", "levels", "const", "special"]
SCALE = max(1, int(os.environ.get("DCPTOPK_FUZZ_SCALE", "1")))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()


def _count(rng, lo=1, hi=16384):
    return int(np.clip(np.exp(rng.uniform(np.log(lo), np.log(hi + 1))), lo, hi))


def _k(rng, c):
    r = rng.random()
    if r < 0.25:
        k = int(rng.integers(1, 65))
    elif r < 0.5:
        k = max(1, c - int(rng.integers(0, 4)))
    elif r < 0.6:
        k = c + int(rng.integers(1, 100))
    else:
        k = int(rng.integers(1, c + 1))
    return min(k, B.MAX_CANDIDATES)


def _gathered(rng, c, k, seed):
    rows = int(rng.integers(1, 7))
    dist = DISTS[int(rng.integers(0, len(DISTS)))]
    pad = float(rng.choice([0.0, 0.0, 0.3, 0.9]))
    repeat = bool(rng.random() < 0.2)
    span = int(rng.integers(1, 64)) if repeat else None
    return W.random_gathered(rows, c, k, seed=seed, dist=dist, pad_frac=pad, repeat_ids=repeat, id_span=span)


def _compare(gb, gi, scores, ids, k, label):
    os_, oi = O.select(scores, ids, k)
    ob = os_.view(np.uint32)
    if not (np.array_equal(gb, ob) and np.array_equal(gi, oi)):
        bad = np.nonzero(~((gb == ob).all(1) & (gi == oi).all(1)))[0]
        raise AssertionError(f"{label}: {len(bad)} rows differ, first {int(bad[0])}")


@pytest.mark.parametrize("block", range(24 * SCALE))
def test_select_random_shapes(block):
    rng = np.random.default_rng(7000 + block)
    for case in range(25):
        c = _count(rng)
        k = _k(rng, c)
        g = _gathered(rng, c, k, seed=int(rng.integers(1 << 30)))
        misalign = bool(rng.random() < 0.25)
        label = f"select block {block} case {case}: {g.name} misalign={misalign}"
        print(label, flush=True)
        gb, gi = gpu_select(g.scores, g.ids, k, guard=1, misalign=misalign)
        _compare(gb, gi, g.scores, g.ids, k, label)


@pytest.mark.parametrize("block", range(6 * SCALE))
def test_split_random_shapes(block):
    rng = np.random.default_rng(7100 + block)
    for case in range(20):
        parts = int(rng.integers(1, 9))
        c = _count(rng, 1, 8192 * parts if parts < 2 else 16384)
        k = _k(rng, c)
        g = _gathered(rng, c, k, seed=int(rng.integers(1 << 30)))
        label = f"split block {block} case {case}: {g.name} parts={parts}"
        print(label, flush=True)
        gb, gi = gpu_select(g.scores, g.ids, k, guard=1, split_parts=parts)
        _compare(gb, gi, g.scores, g.ids, k, label)


@pytest.mark.parametrize("block", range(3 * SCALE))
def test_local_random_shapes(block):
    rng = np.random.default_rng(7200 + block)
    for case in range(30):
        cols = _count(rng)
        k = _k(rng, cols)
        rows = int(rng.integers(1, 7))
        dist = ["normal", "levels", "special"][int(rng.integers(0, 3))]
        lengths = bool(rng.random() < 0.5)
        d = W.local(rows=rows, num_cols=cols, k=k, seed=int(rng.integers(1 << 30)), dist=dist, with_lengths=lengths)
        label = f"local block {block} case {case}: {d.name} lengths={lengths}"
        print(label, flush=True)
        os_, oi = B.local_topk(to_dev(d.scores), d.k, lengths=to_dev(d.lengths) if lengths else None)
        torch.cuda.synchronize()
        ws, wi = O.local_topk(d.scores, d.k, d.lengths if lengths else None)
        assert np.array_equal(os_.cpu().numpy().view(np.uint32), ws.view(np.uint32)), label
        assert np.array_equal(oi.cpu().numpy(), wi), label


@pytest.mark.parametrize("block", range(3 * SCALE))
def test_fused_random_shapes(block):
    rng = np.random.default_rng(7300 + block)
    for case in range(20):
        dcp = int(rng.integers(1, 17))
        local_k = 64 * int(rng.integers(1, 16384 // (64 * dcp) + 1))
        rows = int(rng.integers(1, 7))
        k = _k(rng, dcp * local_k)
        scores = (W.TIE_LEVELS[rng.integers(0, 16, size=(dcp, rows, local_k))] if rng.random() < 0.5
                  else rng.standard_normal((dcp, rows, local_k), dtype=np.float32))
        idx = np.stack([W.distinct_per_row(rng, rows, local_k, 4 * local_k) for _ in range(dcp)])
        idx = np.where(rng.random(idx.shape) < float(rng.choice([0.0, 0.1, 0.6])), np.int32(-1), idx).astype(np.int32)
        starts = rng.integers(0, 1 << 20, size=(dcp, rows), dtype=np.int32)
        offs = (np.arange(dcp) * (1 << 22)).astype(np.int32)
        label = f"fused block {block} case {case}: dcp={dcp} local_k={local_k} rows={rows} k={k}"
        print(label, flush=True)
        out = B.merge_fused([to_dev(scores[r]) for r in range(dcp)], [to_dev(idx[r]) for r in range(dcp)],
                            [to_dev(starts[r]) for r in range(dcp)], [int(x) for x in offs], k)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        want_s, want_i = O.merge(scores, idx, starts, offs, k)
        assert np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)), label
        assert np.array_equal(o[..., 1], want_i), label
