"""Race stress: the selection under adversarial wave timing.

vLLM PR #47348 (review comment) describes the race a radix selector must
avoid: a threshold broadcast through shared memory that is cleared for the next
phase before every wave has read it, so that late waves drop every tied
candidate.  These tests run the stress build of the library
(``DCPTOPK_RACE_STRESS=1``), in which every odd wave sleeps for tens of
microseconds after each workgroup barrier.  The even waves then move on to the
next phase's writes, clears and buffer reuse long before the odd waves read
what the barrier published, so a buffer reused without a barrier after its last
read would give a wrong result.  Every case must still match the oracle bit
for bit: the tie-heavy workload on 256 rows, the large workload, padding-heavy
rows, the register passes (one shared key), full duplicates (the position
rank), 32 items per thread, 1024 threads x 16 items (rows past 8192
candidates), the fused merge, the local top-K and the split-row select.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_select_parity, gpu_select, to_dev
from oracle import stable_topk as O
from stable_top_selection_amd import binding as B
from stable_top_selection_amd import build as BLD
from stable_top_selection_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _stress_library():
    """Every binding call in this module goes through the stress build."""
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    product = B.load_library()
    B._lib = B.open_library(BLD.STRESS_LIB_PATH)
    yield
    B._lib = product


def _select(g, label):
    print(f"[race stress] {label}: {g.name} rows={g.rows} C={g.num_cand} k={g.k}", flush=True)
    assert_select_parity(g.scores, g.ids, g.k, f"race stress {label}", guard=1)


@pytest.mark.parametrize("seed", [40, 41])
def test_tie_heavy_rows(seed):
    _select(W.tie_heavy(rows=256, seed=seed), "tie-heavy")


def test_large_workload():
    _select(W.large(), "large")


def test_padding_heavy_rows():
    _select(W.short_context(), "short context")


@pytest.mark.parametrize("rows,c,k,dist,kw", [
    (8, 8192, 2048, "const", {}),                                     # one key: register passes
    (8, 8192, 2048, "const", {"id_span": 64, "repeat_ids": True}),  # full duplicates: position rank
    (4, 16384, 5000, "levels", {}),                                 # 32 items per thread
    (5, 2049, 1000, "levels", {}),
    (3, 1025, 1, "special", {}),
    (3, 12000, 3000, "levels", {}),                                 # 1024 threads x 16 items (partial row)
])
def test_ragged_and_degenerate(rows, c, k, dist, kw):
    _select(W.random_gathered(rows, c, k, seed=900 + c + k, dist=dist, **kw), f"{dist} {kw}")


@pytest.mark.parametrize("make", [lambda: W.block_heads(32, 601, heads_high=False),
                                  lambda: W.block_heads(32, 602, heads_high=True),
                                  lambda: W.crowded(32, 603, tie=False), lambda: W.crowded(32, 604, tie=True)],
                         ids=["block_heads_low", "block_heads_high", "crowded_sub_bin", "crowded_tie"])
def test_adversarial_rows(make):
    """Rows whose first chunks are unlike the rest, a crowded threshold sub-bin
    (list passes past the first) and a crowded tie (id passes)."""
    _select(make(), "adversarial rows")


def test_fused_merge():
    sh = W.fused()
    print(f"[race stress] fused merge {sh.name}", flush=True)
    sc = [to_dev(sh.scores[r]) for r in range(sh.dcp)]
    ix = [to_dev(sh.local_idx[r]) for r in range(sh.dcp)]
    rs = [to_dev(sh.row_starts[r]) for r in range(sh.dcp)]
    out = B.merge_fused(sc, ix, rs, [int(x) for x in sh.rank_offsets], sh.k)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    want_s, want_i = O.merge(sh.scores, sh.local_idx, sh.row_starts, sh.rank_offsets, sh.k)
    assert np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)) and np.array_equal(o[..., 1], want_i)


def test_fused_merge_partial_32_item_rows():
    """DCP 6 x local K 2048 = 12288 candidates: the partial-row 32-item kernel,
    tie-heavy scores with invalid slots."""
    rng = np.random.default_rng(6144)
    dcp, rows, lk, k = 6, 16, 2048, 2048
    scores = W.TIE_LEVELS[rng.integers(0, 16, size=(dcp, rows, lk))]
    idx = np.stack([W.distinct_per_row(rng, rows, lk, 4096) for _ in range(dcp)])
    idx = np.where(rng.random(idx.shape) < 0.05, np.int32(-1), idx).astype(np.int32)
    starts = rng.integers(0, 131072, size=(dcp, rows), dtype=np.int32)
    offs = (np.arange(dcp) * 135168).astype(np.int32)
    print("[race stress] fused merge dcp 6 x 2048, levels", flush=True)
    out = B.merge_fused([to_dev(scores[r]) for r in range(dcp)], [to_dev(idx[r]) for r in range(dcp)],
                        [to_dev(starts[r]) for r in range(dcp)], [int(x) for x in offs], k)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    want_s, want_i = O.merge(scores, idx, starts, offs, k)
    assert np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)) and np.array_equal(o[..., 1], want_i)


def test_local_topk():
    d = W.local(rows=64, dist="levels", with_lengths=True)
    print(f"[race stress] local top-K {d.name}", flush=True)
    os_, oi = B.local_topk(to_dev(d.scores), d.k, lengths=to_dev(d.lengths))
    torch.cuda.synchronize()
    ws, wi = O.local_topk(d.scores, d.k, d.lengths)
    assert np.array_equal(os_.cpu().numpy().view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(oi.cpu().numpy(), wi)


@pytest.mark.parametrize("make,parts", [(lambda: W.decode(16), 4), (lambda: W.tie_heavy(rows=16, seed=42), 8),
                                        (lambda: W.random_gathered(8, 8192, 2048, seed=943, dist="const",
                                                                   id_span=64, repeat_ids=True), 4)],
                         ids=["decode_16_parts4", "tie_heavy_parts8", "duplicates_parts4"])
def test_split_rows(make, parts):
    """The split-row select: its workgroup barriers under delayed waves, with
    the row barriers between workgroups in between."""
    g = make()
    print(f"[race stress] split rows {g.name} parts={parts}", flush=True)
    gb, gi = gpu_select(g.scores, g.ids, g.k, split_parts=parts)
    os_, oi = O.select(g.scores, g.ids, g.k)
    assert np.array_equal(gb, os_.view(np.uint32)) and np.array_equal(gi, oi)


def test_local_topk_long_rows():
    """Rows of more than 8192 columns with per-row lengths: the 1024-thread
    dense kernel."""
    d = W.local(rows=8, num_cols=12288, k=2048, dist="levels", with_lengths=True)
    print(f"[race stress] local top-K {d.name}", flush=True)
    os_, oi = B.local_topk(to_dev(d.scores), d.k, lengths=to_dev(d.lengths))
    torch.cuda.synchronize()
    ws, wi = O.local_topk(d.scores, d.k, d.lengths)
    assert np.array_equal(os_.cpu().numpy().view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(oi.cpu().numpy(), wi)
