"""GPU parity of dcp_topk_local (each rank's local top-K of its indexer
scores) with the CPU oracle, and of the two-stage pipeline local top-K ->
fused merge with the oracle's merge."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, to_dev
from oracle import stable_topk as O
from stable_top_selection_amd import binding as B
from stable_top_selection_amd import workloads as W

pytestmark = pytest.mark.gpu

PAD_BITS = 0xFF800000


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()


def _gpu_local(scores, k, lengths=None, in_pad=0, in_shift=0, out_pad=0, guard=2):
    """Local top-K on the GPU.  ``in_pad`` extra columns per input row (a row
    stride wider than the row), ``in_shift`` elements before the first row (4
    bytes off an 8-byte boundary when odd), ``out_pad`` extra columns per
    output row; ``guard`` canary rows around each output must survive."""
    rows, cols = scores.shape
    flat = torch.full((in_shift + rows * (cols + in_pad) + 1,), 7.0, dtype=torch.float32, device=DEV)
    src = flat[in_shift:in_shift + rows * (cols + in_pad)].view(rows, cols + in_pad)[:, :cols]
    src.copy_(to_dev(scores))
    width = k + out_pad
    big_s = torch.full((rows + 2 * guard, width), -5.5, dtype=torch.float32, device=DEV)
    big_i = torch.full((rows + 2 * guard, width), 0x0BADF00D, dtype=torch.int32, device=DEV)
    os_ = big_s[guard:guard + rows, :k]
    oi = big_i[guard:guard + rows, :k]
    lens = to_dev(lengths) if lengths is not None else None
    B.local_topk(src, k, lengths=lens, out_scores=os_, out_idx=oi)
    torch.cuda.synchronize()
    gs, gi = big_s.cpu().numpy(), big_i.cpu().numpy()
    keep = np.ones((rows + 2 * guard, width), bool)
    keep[guard:guard + rows, :k] = False
    assert np.all(gs[keep] == -5.5) and np.all(gi[keep] == 0x0BADF00D), "wrote outside the outputs"
    return gs[guard:guard + rows, :k].view(np.uint32), gi[guard:guard + rows, :k]


def _parity(scores, k, lengths=None, label="", **kw):
    print(f"[local parity] {label}", flush=True)
    gb, gi = _gpu_local(scores, k, lengths, **kw)
    ws, wi = O.local_topk(scores, k, lengths)
    wb = ws.view(np.uint32)
    ok = (gb == wb).all(1) & (gi == wi).all(1)
    if not ok.all():
        r = int(np.nonzero(~ok)[0][0])
        c = int(np.nonzero((gb[r] != wb[r]) | (gi[r] != wi[r]))[0][0])
        raise AssertionError(f"{label}: {np.count_nonzero(~ok)} rows differ; row {r} col {c}: "
                             f"gpu ({gb[r, c]:#x}, {gi[r, c]}) oracle ({wb[r, c]:#x}, {wi[r, c]})")


@pytest.mark.parametrize("rows", [1, 8, 32, 64, 256])
def test_local_pages_shape(rows):
    """2048 of 4096 local score columns per row (the decode shape measured on
    PR #50009, rows 1 to 64, and 256)."""
    d = W.local(rows=rows)
    _parity(d.scores, d.k, label=d.name)


@pytest.mark.parametrize("dist", ["levels", "special"])
def test_local_ties_and_specials(dist):
    d = W.local(rows=24, dist=dist)
    _parity(d.scores, d.k, label=d.name)


def test_local_lengths():
    """Per-row lengths U[0, 4096]: rows shorter than k keep every valid column
    and pad with (-inf, -1); explicit 0, negative and past-the-end lengths."""
    d = W.local(rows=40, with_lengths=True)
    lens = d.lengths.copy()
    lens[:4] = [0, -9, 4096 + 7, 2048]
    _parity(d.scores, d.k, lens, label="lengths")
    gb, gi = _gpu_local(d.scores, d.k, lens)
    assert np.all(gb[:2] == PAD_BITS) and np.all(gi[:2] == -1)


@pytest.mark.parametrize("rows,cols,k", [(3, 1, 1), (5, 63, 17), (4, 100, 150), (6, 513, 512), (2, 4097, 2048),
                                         (3, 2047, 2), (2, 16384, 2048), (3, 12000, 9000), (7, 256, 256),
                                         (9, 8191, 4096)])
def test_local_ragged(rows, cols, k):
    d = W.local(rows=rows, num_cols=cols, k=k, dist="levels" if cols % 3 == 0 else "normal")
    _parity(d.scores, k, label=f"ragged {rows}x{cols} k={k}")


@pytest.mark.parametrize("in_pad,in_shift,out_pad", [(6, 0, 0), (5, 1, 3), (0, 1, 0), (2, 0, 9), (0, 2, 0), (4, 0, 1)])
def test_local_strides_and_alignment(in_pad, in_shift, out_pad):
    """Row strides wider than the rows, and inputs off a 16-byte boundary:
    4-byte loads for an odd stride or a 4-byte offset, 8-byte loads for an
    even stride that is not a multiple of 4 or an 8-byte offset, 16-byte
    loads otherwise."""
    d = W.local(rows=12, num_cols=1000, k=300, dist="levels")
    _parity(d.scores, d.k, label=f"strides {in_pad}/{in_shift}/{out_pad}", in_pad=in_pad, in_shift=in_shift,
            out_pad=out_pad)


def test_local_then_fused_merge_is_global_topk():
    """The whole two-stage pipeline on the GPU: local top-K of 4 ranks' 4096
    columns, then the fused merge, against the oracle applied to the same two
    stages."""
    rows, dcp, k = 32, 4, 2048
    ranks = [W.local(rows=rows, seed=100 + r) for r in range(dcp)]
    starts = np.random.default_rng(5).integers(0, 131072, size=rows, dtype=np.int32)
    offs = [r * W.PREFILL_RANK_STRIDE for r in range(dcp)]
    sc, ix = [], []
    for d in ranks:
        s, i = B.local_topk(to_dev(d.scores), k)
        sc.append(s)
        ix.append(i)
    rs = [to_dev(starts)] * dcp
    out = B.merge_fused(sc, ix, rs, offs, k)
    torch.cuda.synchronize()
    loc = [O.local_topk(d.scores, k) for d in ranks]
    ws, wi = O.merge(np.stack([l[0] for l in loc]), np.stack([l[1] for l in loc]), np.stack([starts] * dcp),
                     np.array(offs, np.int32), k)
    o = out.cpu().numpy()
    assert np.array_equal(o[..., 0].view(np.uint32), ws.view(np.uint32)) and np.array_equal(o[..., 1], wi)


def test_local_errors():
    s = torch.zeros((4, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(B.DcpTopkError) as e:
        B.local_topk(torch.zeros((2, 16385), dtype=torch.float32, device=DEV), 8)
    assert e.value.status == B.EUNSUPPORTED
    with pytest.raises(B.DcpTopkError) as e:
        B.local_topk(s, 16385)
    assert e.value.status == B.EUNSUPPORTED
    alias_i = s.view(torch.int32)[:, :8]  # index output inside the scores
    out_s = torch.empty((4, 64), dtype=torch.float32, device=DEV)[:, :8]
    with pytest.raises(B.DcpTopkError) as e:
        B.local_topk(s, 8, out_scores=out_s, out_idx=alias_i)
    assert e.value.status == B.EINVAL


def test_local_max_rows():
    """DCP_TOPK_MAX_ROWS rows (4,194,303) of 3 columns with per-row lengths, k 2:
    the largest grid one launch takes.  200,000 seeded rows are checked
    against the oracle; one row more is refused before any launch."""
    rows = B.MAX_ROWS
    rng = np.random.default_rng(4343)
    scores = rng.standard_normal((rows, 3), dtype=np.float32)
    lengths = rng.integers(-1, 5, size=rows, dtype=np.int32)
    os_, oi = B.local_topk(to_dev(scores), 2, lengths=to_dev(lengths))
    torch.cuda.synchronize()
    pick = np.sort(rng.choice(rows, 200000, replace=False))
    ws, wi = O.local_topk(scores[pick], 2, lengths[pick])
    assert np.array_equal(os_.cpu().numpy()[pick].view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(oi.cpu().numpy()[pick], wi)
    del os_, oi
    big = torch.zeros((rows + 1, 3), dtype=torch.float32, device=DEV)
    with pytest.raises(B.DcpTopkError) as e:
        B.local_topk(big, 2)
    assert e.value.status == B.EUNSUPPORTED
    del big
    torch.cuda.empty_cache()


def test_local_graph_replay_with_changing_inputs():
    """Captured into a HIP graph once; before each replay the scores and the
    per-row lengths are overwritten in place (eager copies, a synchronisation
    in between): every replay matches the oracle on its own inputs."""
    rows, cols, k = 32, 4096, 2048
    scores = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
    lengths = torch.empty((rows,), dtype=torch.int32, device=DEV)
    os_ = torch.empty((rows, k), dtype=torch.float32, device=DEV)
    oi = torch.empty((rows, k), dtype=torch.int32, device=DEV)
    d0 = W.local(rows=rows, num_cols=cols, k=k, seed=90, with_lengths=True)
    scores.copy_(to_dev(d0.scores))
    lengths.copy_(to_dev(d0.lengths))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.local_topk(scores, k, lengths=lengths, out_scores=os_, out_idx=oi)  # outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.local_topk(scores, k, lengths=lengths, out_scores=os_, out_idx=oi)
    for seed, dist in ((91, "normal"), (92, "levels"), (93, "special")):
        d = W.local(rows=rows, num_cols=cols, k=k, seed=seed, dist=dist, with_lengths=True)
        scores.copy_(to_dev(d.scores))
        lengths.copy_(to_dev(d.lengths))
        os_.fill_(0.0)
        g.replay()
        torch.cuda.synchronize()
        ws, wi = O.local_topk(d.scores, k, d.lengths)
        assert np.array_equal(os_.cpu().numpy().view(np.uint32), ws.view(np.uint32)), f"replay {seed}"
        assert np.array_equal(oi.cpu().numpy(), wi), f"replay {seed}"
