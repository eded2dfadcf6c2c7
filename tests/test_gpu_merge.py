"""GPU parity of dcp_topk_pack and dcp_topk_merge_chunked with the CPU oracle."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, to_dev
from oracle import stable_topk as O
from stable_top_selection_amd import binding as B
from stable_top_selection_amd import workloads as W

pytestmark = pytest.mark.gpu

INT32_MAX = 2**31 - 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()


def _shards_to_dev(sh):
    return ([to_dev(sh.scores[r]) for r in range(sh.dcp)], [to_dev(sh.local_idx[r]) for r in range(sh.dcp)],
            [to_dev(sh.row_starts[r]) for r in range(sh.dcp)], [int(x) for x in sh.rank_offsets])


def _random_shards(rows, dcp, local_k, seed, invalid_frac=0.0, span=4096):
    rng = np.random.default_rng(seed)
    scores = rng.standard_normal((dcp, rows, local_k), dtype=np.float32)
    if local_k <= span:
        idx = np.stack([W.distinct_per_row(rng, rows, local_k, span) for _ in range(dcp)])
    else:
        idx = rng.integers(0, span, size=(dcp, rows, local_k), dtype=np.int32)
    if invalid_frac:
        idx = np.where(rng.random(idx.shape) < invalid_frac, np.int32(-1), idx).astype(np.int32)
    starts = rng.integers(0, 131072, size=(dcp, rows), dtype=np.int32)
    offs = (np.arange(dcp) * (131072 + span)).astype(np.int32)
    return W.LocalShards("random", scores, idx, starts, offs, k=0)


@pytest.mark.parametrize("rows,local_k,column,width", [(7, 2048, 2048, 8192), (5, 37, 3, 100), (3, 1, 0, 1),
                                                      (1024, 2048, 0, 2048), (9, 1030, 0, 1030)])
def test_pack_parity(rows, local_k, column, width):
    sh = _random_shards(rows, 1, local_k, seed=rows + local_k, invalid_frac=0.05)
    dst = torch.full((rows, width, 2), 123, dtype=torch.int32, device=DEV)
    B.pack(to_dev(sh.scores[0]), to_dev(sh.local_idx[0]), to_dev(sh.row_starts[0]), 777, dst, column=column)
    torch.cuda.synchronize()
    want_s, want_i = O.pack(sh.scores[0], sh.local_idx[0], sh.row_starts[0], 777)
    o = dst.cpu().numpy()
    assert np.array_equal(o[:, column:column + local_k, 0].view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(o[:, column:column + local_k, 1], want_i)
    untouched = np.ones(width, bool)
    untouched[column:column + local_k] = False
    assert np.all(o[:, untouched] == 123), "pack wrote outside its columns"


def test_pack_max_rows():
    """dcp_topk_pack over DCP_TOPK_MAX_ROWS rows (4,194,303) of 2 slots into
    columns 1-2 of a 4-column buffer, with invalid slots: every row against
    the oracle; one row more is refused before any launch."""
    rows, local_k, width = B.MAX_ROWS, 2, 4
    rng = np.random.default_rng(4444)
    scores = rng.standard_normal((rows, local_k), dtype=np.float32)
    idx = rng.integers(-1, 4096, size=(rows, local_k), dtype=np.int32)
    starts = rng.integers(0, 1 << 20, size=rows, dtype=np.int32)
    dst = torch.full((rows, width, 2), 123, dtype=torch.int32, device=DEV)
    B.pack(to_dev(scores), to_dev(idx), to_dev(starts), 5 << 22, dst, column=1)
    torch.cuda.synchronize()
    want_s, want_i = O.pack(scores, idx, starts, 5 << 22)
    o = dst.cpu().numpy()
    assert np.array_equal(o[:, 1:3, 0].view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(o[:, 1:3, 1], want_i)
    assert np.all(o[:, 0] == 123) and np.all(o[:, 3] == 123), "pack wrote outside its columns"
    del dst
    one_more = torch.zeros((rows + 1, local_k), dtype=torch.float32, device=DEV)
    one_more_idx = torch.zeros((rows + 1, local_k), dtype=torch.int32, device=DEV)
    one_more_starts = torch.zeros((rows + 1,), dtype=torch.int32, device=DEV)
    one_more_dst = torch.zeros((rows + 1, local_k, 2), dtype=torch.int32, device=DEV)
    with pytest.raises(B.DcpTopkError) as e:
        B.pack(one_more, one_more_idx, one_more_starts, 0, one_more_dst)
    assert e.value.status == B.EUNSUPPORTED
    del one_more, one_more_idx, one_more_starts, one_more_dst
    torch.cuda.empty_cache()


def test_pack_wraps_and_marks_invalid():
    scores = torch.tensor([[1.5, -2.0, 3.0, 4.0]], dtype=torch.float32, device=DEV)
    idx = torch.tensor([[2**31 - 10, -1, 0, -7]], dtype=torch.int32, device=DEV)
    starts = torch.tensor([20], dtype=torch.int32, device=DEV)
    dst = torch.zeros((1, 4, 2), dtype=torch.int32, device=DEV)
    B.pack(scores, idx, starts, 5, dst)
    o = dst.cpu().numpy()
    want_s, want_i = O.pack(scores.cpu().numpy(), idx.cpu().numpy(), starts.cpu().numpy(), 5)
    assert np.array_equal(o[..., 1], want_i) and np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32))
    assert o[0, 1, 1] == INT32_MAX and o[0, 3, 1] == INT32_MAX


def _merge_parity(sh, k, label):
    sc, ix, rs, offs = _shards_to_dev(sh)
    out = B.merge_chunked(sc, ix, rs, offs, k)
    torch.cuda.synchronize()
    want_s, want_i = O.merge(sh.scores, sh.local_idx, sh.row_starts, sh.rank_offsets, k)
    o = out.cpu().numpy()
    ok_rows = (o[..., 0].view(np.uint32) == want_s.view(np.uint32)).all(1) & (o[..., 1] == want_i).all(1)
    assert ok_rows.all(), f"{label}: {np.count_nonzero(~ok_rows)} rows differ, first {np.nonzero(~ok_rows)[0][0]}"


@pytest.mark.parametrize("rows", [1, 5, 1024, 1025, 2 * 1024 + 5])
def test_merge_chunked_prefill_shape(rows):
    """DCP 4 x local K 2048, K 2048, across chunk boundaries (2*1024+5 rows is
    the row count of PR #59367's chunk-walk test)."""
    sh = W.prefill(rows=rows, seed=50 + rows)
    print(f"[merge parity] T={rows} digest={sh.digest()}", flush=True)
    _merge_parity(sh, 2048, f"prefill T={rows}")


def test_merge_chunked_full_prefill():
    """The prefill workload at full size: T = 8192 rows in 8 chunks."""
    sh = W.prefill()
    print(f"[merge parity] {sh.name} digest={sh.digest()}", flush=True)
    _merge_parity(sh, sh.k, sh.name)


def test_merge_chunked_past_the_single_launch_row_limit():
    """The chunked merge launches 1024 rows at a time, so it takes more rows
    than one launch may: 4,194,816 rows (DCP_TOPK_MAX_ROWS + 513, a last chunk
    of 512) of DCP 1 x local K 64, k 5, from a seeded 4096-row block with
    invalid slots tiled on the device.  Whole repeats of the block and the
    last, partial one are checked against the oracle's result for the block."""
    block_rows, local_k, k = 4096, 64, 5
    rows = B.MAX_ROWS + 513
    reps = -(-rows // block_rows)
    sh = _random_shards(block_rows, 1, local_k, seed=4646, invalid_frac=0.05)
    want_s, want_i = O.merge(sh.scores, sh.local_idx, sh.row_starts, sh.rank_offsets, k)
    want = np.stack([want_s.view(np.int32), want_i], axis=-1)
    sc = to_dev(sh.scores[0]).repeat(reps, 1)[:rows]
    ix = to_dev(sh.local_idx[0]).repeat(reps, 1)[:rows]
    rs = to_dev(sh.row_starts[0]).repeat(reps)[:rows]
    out = B.merge_chunked([sc], [ix], [rs], [int(sh.rank_offsets[0])], k)
    torch.cuda.synchronize()
    assert out.shape[0] == rows > B.MAX_ROWS
    for r in (0, reps // 2, reps - 2):
        got = out[r * block_rows:(r + 1) * block_rows].cpu().numpy()
        assert np.array_equal(got, want), f"block repeat {r} differs"
    tail = rows - (reps - 1) * block_rows
    assert np.array_equal(out[(reps - 1) * block_rows:].cpu().numpy(), want[:tail]), "the last, partial repeat differs"
    del sc, ix, rs, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("rows,dcp,local_k,k", [(37, 3, 100, 50), (20, 9, 64, 100), (11, 2, 7, 20),
                                               (1030, 4, 33, 1), (6, 16, 1024, 2048), (4, 4, 0, 3)])
def test_merge_chunked_ragged(rows, dcp, local_k, k):
    sh = _random_shards(rows, dcp, local_k, seed=rows * dcp + local_k, invalid_frac=0.1, span=max(local_k, 128))
    _merge_parity(sh, k, f"ragged rows={rows} dcp={dcp} local_k={local_k} k={k}")


def test_merge_equals_pack_then_select():
    """The driver equals the two public calls composed on the caller's side."""
    sh = W.prefill(rows=300, seed=9)
    sc, ix, rs, offs = _shards_to_dev(sh)
    gathered = torch.empty((300, 4 * 2048, 2), dtype=torch.int32, device=DEV)
    for r in range(4):
        B.pack(sc[r], ix[r], rs[r], offs[r], gathered, column=r * 2048)
    a = B.select(gathered, 2048)
    b = B.merge_chunked(sc, ix, rs, offs, 2048)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_merge_workspace_errors():
    sh = W.prefill(rows=8, seed=1, local_k=64)
    sc, ix, rs, offs = _shards_to_dev(sh)
    need = B.merge_workspace_bytes(8, 4, 64)
    assert need == O.merge_workspace_bytes(8, 4, 64)
    small = torch.empty(need - 8, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.DcpTopkError) as e:
        B.merge_chunked(sc, ix, rs, offs, 16, workspace=small)
    assert e.value.status == B.EWORKSPACE
    big = torch.empty(need + 512, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.DcpTopkError) as e:  # 8 bytes past a 256-byte boundary
        B.merge_chunked(sc, ix, rs, offs, 16, workspace=big[8:8 + need])
    assert e.value.status == B.EWORKSPACE


def test_merge_chunked_workspace_canaries():
    """Guard bytes just before the workspace and just past its ``need`` bytes
    survive the chunked merge (T = 2*1024+5 rows: three chunks, the last one
    short)."""
    rows = 2 * 1024 + 5
    sh = W.prefill(rows=rows, seed=2053)
    sc, ix, rs, offs = _shards_to_dev(sh)
    need = B.merge_workspace_bytes(rows, sh.dcp, sh.local_k)
    guard = 4096
    ws_all = torch.full((guard + need + guard,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = ws_all[guard:guard + need]
    assert ws.data_ptr() % B.WORKSPACE_ALIGN == 0
    out = B.merge_chunked(sc, ix, rs, offs, sh.k, workspace=ws)
    torch.cuda.synchronize()
    g = ws_all.cpu().numpy()
    assert np.all(g[:guard] == 0xA5), "wrote before the workspace"
    assert np.all(g[guard + need:] == 0xA5), "wrote past the workspace's required bytes"
    want_s, want_i = O.merge(sh.scores, sh.local_idx, sh.row_starts, sh.rank_offsets, sh.k)
    o = out.cpu().numpy()
    assert np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)) and np.array_equal(o[..., 1], want_i)


def test_merge_chunked_graph_replay_changing_inputs():
    """The chunked merge (T = 1024+37 rows: two chunks through one workspace)
    captured once into a HIP graph, then replayed three times with new inputs
    copied into the captured buffers between replays (PR #47348, Summary: the
    merge is graph-capturable; PR #50009, Validation: replay with changing
    inputs).  Every replay matches the oracle on that replay's inputs."""
    rows = 1024 + 37
    shards = [W.prefill(rows=rows, seed=700 + i) for i in range(4)]
    sc, ix, rs, offs = _shards_to_dev(shards[0])
    need = B.merge_workspace_bytes(rows, 4, 2048)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.empty((rows, 2048, 2), dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.merge_chunked(sc, ix, rs, offs, 2048, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.merge_chunked(sc, ix, rs, offs, 2048, workspace=ws, out=out)
    for rep, sh in enumerate(shards[1:] + shards[:1]):
        for r in range(4):
            sc[r].copy_(to_dev(sh.scores[r]))
            ix[r].copy_(to_dev(sh.local_idx[r]))
            rs[r].copy_(to_dev(sh.row_starts[r]))
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want_s, want_i = O.merge(sh.scores, sh.local_idx, sh.row_starts, sh.rank_offsets, 2048)
        o = out.cpu().numpy()
        assert np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)), f"replay {rep}: scores"
        assert np.array_equal(o[..., 1], want_i), f"replay {rep}: ids"
