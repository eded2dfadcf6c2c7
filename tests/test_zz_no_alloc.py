"""dcp_topk_merge_chunked_static, the chunked merge for callers that cannot
allocate: its chunk workspace is the library's static per-GPU buffer.  Its
output must equal dcp_topk_merge_chunked's (and the oracle's) bit for bit on
two calls in a row, the second with a smaller input, and under HIP graph
capture; shapes that need more than the buffer are refused before anything
is enqueued."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, to_dev
from oracle import stable_topk as O
from stable_top_selection_amd import binding as B
from stable_top_selection_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()


def _dev(sh):
    return ([to_dev(sh.scores[r]) for r in range(sh.dcp)], [to_dev(sh.local_idx[r]) for r in range(sh.dcp)],
            [to_dev(sh.row_starts[r]) for r in range(sh.dcp)], [int(x) for x in sh.rank_offsets])


def _check(sh, got, label):
    want_s, want_i = O.merge(sh.scores, sh.local_idx, sh.row_starts, sh.rank_offsets, sh.k)
    o = got.cpu().numpy()
    assert np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)), f"{label}: scores differ"
    assert np.array_equal(o[..., 1], want_i), f"{label}: ids differ"


def test_two_calls_in_a_row_match_the_workspace_merge():
    """A 3-chunk merge (DCP 4 x 2048, T = 2*1024+5), then a smaller one (DCP 3
    x 1024, T = 300, invalid slots): each equals dcp_topk_merge_chunked's
    output on the same inputs, bit for bit, and the oracle's."""
    big = W.prefill(rows=2 * 1024 + 5, seed=811)
    small = W.prefill(rows=300, seed=812, dcp=3, local_k=1024, invalid_frac=0.05)
    for label, sh in (("first call, T=2053 dcp 4 x 2048", big), ("second call, T=300 dcp 3 x 1024", small)):
        print(f"[no-alloc] {label}", flush=True)
        args = _dev(sh)
        got = B.merge_chunked_static(*args, sh.k)
        ref = B.merge_chunked(*args, sh.k)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{label}: differs from dcp_topk_merge_chunked"
        _check(sh, got, label)


def test_graph_capture_and_replay():
    """Captured into a HIP graph (where the caller could not allocate) and
    replayed twice with new inputs copied in and eager work between replays."""
    shards = [W.prefill(rows=1024 + 9, seed=820 + i) for i in range(3)]
    sc, ix, rs, offs = _dev(shards[0])
    out = torch.empty((1024 + 9, 2048, 2), dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.merge_chunked_static(sc, ix, rs, offs, 2048, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.merge_chunked_static(sc, ix, rs, offs, 2048, out=out)
    for rep, sh in enumerate(shards[1:]):
        print(f"[no-alloc] graph replay {rep}", flush=True)
        for r in range(4):
            sc[r].copy_(to_dev(sh.scores[r]))
            ix[r].copy_(to_dev(sh.local_idx[r]))
            rs[r].copy_(to_dev(sh.row_starts[r]))
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check(sh, out, f"replay {rep}")


def test_shapes_beyond_the_buffer_are_refused():
    """1024 rows of DCP 4 x 4096 need 128 MiB of workspace: refused with
    DCP_TOPK_ESCRATCH; 1023 rows of DCP 2 x 4096 (64 MiB - 64 KiB) fit."""
    sh = W.prefill(rows=1024, seed=830, dcp=4, local_k=4096)
    with pytest.raises(B.DcpTopkError) as e:
        B.merge_chunked_static(*_dev(sh), 2048)
    assert e.value.status == B.ESCRATCH
    fits = W.prefill(rows=1023, seed=831, dcp=2, local_k=4096)
    assert B.merge_workspace_bytes(1023, 2, 4096) <= B.STATIC_SCRATCH_BYTES
    args = _dev(fits)
    got = B.merge_chunked_static(*args, 2048)
    torch.cuda.synchronize()
    assert torch.equal(got, B.merge_chunked(*args, 2048))
