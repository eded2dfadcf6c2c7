"""GPU parity on rows built to stress particular steps of the select, through
the gathered select (both load widths), the fused merge and the local top-K:

- block_heads_low / block_heads_high: the first 256 candidates of every
  1024-candidate block come from another score distribution than the rest
  (the first chunk of every wave is unlike its other chunks);
- crowded: the k-th best key falls among 64 near-equal scores inside one
  pass-0 bin, so the threshold needs list passes past the first one (distinct
  keys) or the id tie-break over a crowd of one key;
- k = C / 2 on N(0,1): the threshold sits at the sign change of the keys;
- rows of 12000 candidates (the partial-row 32-item kernels).

Every result must equal the oracle's bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_select_parity, to_dev
from oracle import stable_topk as O
from stable_top_selection_amd import binding as B
from stable_top_selection_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()


CASES = [
    ("block_heads_low", lambda: W.block_heads(16, 501, heads_high=False)),
    ("block_heads_high", lambda: W.block_heads(16, 502, heads_high=True)),
    ("crowded_distinct", lambda: W.crowded(16, 503, tie=False)),
    ("crowded_tie", lambda: W.crowded(16, 504, tie=True)),
    ("half_of_normal", lambda: W.random_gathered(8, 8192, 4096, seed=505, dist="normal")),
    ("block_heads_low_k1000", lambda: W.block_heads(8, 506, heads_high=False, k=1000)),
    ("crowded_12000", lambda: W.crowded(6, 507, tie=False, num_cand=12000)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_select_adversarial_rows(name, make):
    g = make()
    print(f"[adversarial] select {g.name}", flush=True)
    assert_select_parity(g.scores, g.ids, g.k, g.name, guard=1)
    assert_select_parity(g.scores, g.ids, g.k, g.name + " (8-byte loads)", misalign=True)


@pytest.mark.parametrize("name,make", CASES[:4], ids=[c[0] for c in CASES[:4]])
def test_fused_adversarial_rows(name, make):
    """The same rows as 4 ranks of 2048 local slots (ids as local index +
    rank offset), through the fused merge's four-item loads."""
    g = make()
    print(f"[adversarial] fused {g.name}", flush=True)
    dcp, lk = 4, 2048
    scores = np.ascontiguousarray(g.scores.reshape(g.rows, dcp, lk).transpose(1, 0, 2))
    idx = np.ascontiguousarray(np.broadcast_to(np.arange(lk, dtype=np.int32), (dcp, g.rows, lk)))
    starts = np.zeros((dcp, g.rows), np.int32)
    offs = (np.arange(dcp) * lk).astype(np.int32)
    out = B.merge_fused([to_dev(scores[r]) for r in range(dcp)], [to_dev(idx[r]) for r in range(dcp)],
                        [to_dev(starts[r]) for r in range(dcp)], [int(x) for x in offs], g.k)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    want_s, want_i = O.merge(scores, idx, starts, offs, g.k)
    assert np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)) and np.array_equal(o[..., 1], want_i)


@pytest.mark.parametrize("name,make", CASES[:4], ids=[c[0] for c in CASES[:4]])
def test_local_adversarial_rows(name, make):
    """The same rows as dense score rows (ids = columns) through the local
    top-K, with and without per-row lengths."""
    g = make()
    print(f"[adversarial] local {g.name}", flush=True)
    lengths = np.random.default_rng(508).integers(6000, g.num_cand + 1, size=g.rows).astype(np.int32)
    for lens in (None, lengths):
        os_, oi = B.local_topk(to_dev(g.scores), g.k, lengths=None if lens is None else to_dev(lens))
        torch.cuda.synchronize()
        ws, wi = O.local_topk(g.scores, g.k, lens)
        assert np.array_equal(os_.cpu().numpy().view(np.uint32), ws.view(np.uint32))
        assert np.array_equal(oi.cpu().numpy(), wi)
