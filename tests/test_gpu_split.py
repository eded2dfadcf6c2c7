"""Split-row select (dcp_topk_select_split) against the oracle, bit for bit.

PR #50009 (Top-K performance) measures the merge at 1, 8, 32 and 64 decode
rows; there one workgroup per row leaves most compute units idle, so the split
path spreads each row over 2 to 8 workgroups that exchange their pass-0
histograms and threshold-bin items through a workspace.  Every case here must
equal the oracle (and so dcp_topk_select) bit for bit: the decode rows at
every split, tie-heavy rows (id passes, full duplicates across slices),
padding-heavy rows (the padding bin as the threshold bin), ragged candidate
counts with empty trailing slices, the 8-byte load path, workspace reuse
(the counters are back at zero after every call), the k >= C route, and the
residency limit of the cooperative launch.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, gpu_select, to_dev
from oracle import stable_topk as O
from stable_top_selection_amd import binding as B
from stable_top_selection_amd import workloads as W

pytestmark = pytest.mark.gpu


def _parity(scores, ids, k, parts, label, **kw):
    print(f"[split] {label}: rows={scores.shape[0]} C={scores.shape[1]} k={k} parts={parts}", flush=True)
    gb, gi = gpu_select(scores, ids, k, split_parts=parts, **kw)
    os_, oi = O.select(scores, ids, k)
    ob = os_.view(np.uint32)
    if not (np.array_equal(gb, ob) and np.array_equal(gi, oi)):
        bad = np.nonzero(~((gb == ob).all(1) & (gi == oi).all(1)))[0]
        r = int(bad[0])
        col = int(np.nonzero((gb[r] != ob[r]) | (gi[r] != oi[r]))[0][0])
        raise AssertionError(f"{label} parts={parts}: {len(bad)} rows differ; first row {r} col {col}: "
                             f"gpu ({gb[r, col]:#x}, {gi[r, col]}) oracle ({ob[r, col]:#x}, {oi[r, col]})")


@pytest.mark.parametrize("parts", [2, 4, 8])
@pytest.mark.parametrize("rows", [1, 8, 16, 32, 64])
def test_decode_rows(rows, parts):
    g = W.decode(rows)
    _parity(g.scores, g.ids, g.k, parts, g.name, guard=1)


@pytest.mark.parametrize("parts", [1, 3, 4, 8])
def test_tie_heavy_rows(parts):
    g = W.tie_heavy(rows=16)
    _parity(g.scores, g.ids, g.k, parts, g.name)


@pytest.mark.parametrize("parts", [2, 8])
def test_padding_heavy_rows(parts):
    g = W.short_context()
    _parity(g.scores, g.ids, g.k, parts, g.name)


@pytest.mark.parametrize("rows,c,k,dist,kw,parts", [
    (8, 8192, 2048, "const", {}, 4),                                     # one key: the list is every item
    (8, 8192, 2048, "const", {"id_span": 64, "repeat_ids": True}, 4),  # full duplicates in every slice
    (8, 8192, 2048, "const", {"id_span": 64, "repeat_ids": True}, 8),
    (5, 2049, 1000, "levels", {}, 3),                                    # ragged last slice
    (3, 1025, 1, "special", {}, 4),                                      # k = 1, NaN / inf / -0 scores
    (4, 6000, 5999, "normal", {}, 5),                                    # k = C - 1
    (2, 130, 65, "levels", {}, 8),                                       # slices 3..7 empty
    (6, 16384, 2048, "normal", {}, 2),                                   # 8192 per slice
    (6, 16384, 8000, "levels", {}, 4),
])
def test_ragged_and_degenerate(rows, c, k, dist, kw, parts):
    g = W.random_gathered(rows, c, k, seed=1300 + c + k + parts, dist=dist, **kw)
    _parity(g.scores, g.ids, g.k, parts, f"{dist} {kw}")


@pytest.mark.parametrize("make", [lambda: W.block_heads(32, 611, heads_high=True),
                                  lambda: W.crowded(32, 612, tie=False), lambda: W.crowded(32, 613, tie=True)],
                         ids=["block_heads_high", "crowded_sub_bin", "crowded_tie"])
def test_adversarial_rows(make):
    g = make()
    _parity(g.scores, g.ids, g.k, 4, g.name)


def test_eight_byte_loads():
    g = W.decode(16)
    _parity(g.scores, g.ids, g.k, 4, "decode misaligned", misalign=True)


def test_workspace_reuse_leaves_counters_zero():
    """Three calls through one workspace (shapes shrinking, then growing back):
    each matches the oracle, and the counters are zero after each."""
    ws = B.select_split_workspace(64, 8192, 8, DEV)
    for rows, parts, seed in ((64, 8, 31), (8, 4, 32), (64, 8, 33)):
        g = W.random_gathered(rows, 8192, 2048, seed=seed, dist="levels")
        _parity(g.scores, g.ids, g.k, parts, f"reuse seed {seed}", workspace=ws)
        ctrl = ws[:rows * 16].view(torch.int32).cpu().numpy()
        assert not ctrl.any(), f"counters left at {ctrl[ctrl != 0][:8]}"


def test_k_at_least_c_pads_without_the_workspace():
    g = W.random_gathered(4, 1000, 1200, seed=77, dist="normal")
    ws = torch.full((B.select_split_workspace_bytes(4, 1000, 4),), 0xA5, dtype=torch.uint8, device=DEV)
    _parity(g.scores, g.ids, g.k, 4, "k > C", workspace=ws)
    assert bool((ws == 0xA5).all()), "the k >= C route wrote to the workspace"


def test_grid_past_residency_is_unsupported():
    """256 rows x 8 parts is more workgroups than the GPU holds at once: the
    call is refused before anything runs, and a later call still works."""
    g = W.large()
    cand = to_dev(g.interleaved())
    with pytest.raises(B.DcpTopkError) as e:
        B.select_split(cand, g.k, 8)
    assert e.value.status == B.EUNSUPPORTED
    out = B.select(cand, g.k)
    torch.cuda.synchronize()
    want_s, want_i = O.select(g.scores[:2], g.ids[:2], g.k)
    o = out[:2].cpu().numpy()
    assert np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)) and np.array_equal(o[..., 1], want_i)


def test_graph_replay_with_changing_inputs():
    """The cooperative launch captured in a HIP graph: three replays over new
    inputs copied into the captured buffer, with eager work in between; every
    replay matches the oracle and leaves the counters at zero."""
    rows, c, k, parts = 8, 8192, 2048, 4
    cand = torch.zeros((rows, c, 2), dtype=torch.int32, device=DEV)
    out = torch.empty((rows, k, 2), dtype=torch.int32, device=DEV)
    ws = B.select_split_workspace(rows, c, parts, DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.select_split(cand, k, parts, workspace=ws, out=out)  # first launch outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.select_split(cand, k, parts, workspace=ws, out=out)
    for seed in (51, 52, 53):
        g = W.random_gathered(rows, c, k, seed=seed, dist="levels" if seed % 2 else "normal")
        print(f"[split] graph replay seed {seed}", flush=True)
        cand.copy_(to_dev(g.interleaved()))
        B.select(cand, 16)  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        want_s, want_i = O.select(g.scores, g.ids, k)
        assert np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)) and np.array_equal(o[..., 1], want_i)
        assert not ws[:rows * 16].view(torch.int32).cpu().numpy().any()
