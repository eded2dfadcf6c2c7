"""The seeded generators produce the shapes and structure their recipes state."""
import numpy as np

from stable_top_selection_amd import workloads as W


def _check_rank_ranges(g, span):
    for r in range(g.dcp):
        sl = g.ids[:, r * g.local_k:(r + 1) * g.local_k]
        real = sl != W.INT32_MAX
        assert np.all((sl[real] >= r * span) & (sl[real] < (r + 1) * span))
        for row in range(g.rows):
            v = sl[row][real[row]]
            assert len(np.unique(v)) == len(v)


def test_tiny_shape_and_ids():
    g = W.tiny()
    assert (g.rows, g.num_cand, g.k) == (4, 256, 64)
    assert g.scores.dtype == np.float32 and g.ids.dtype == np.int32
    _check_rank_ranges(g, 1024)
    assert W.tiny().digest() == g.digest()


def test_decode_sweep_shapes():
    for rows in (1, 8):
        g = W.decode(rows)
        assert (g.rows, g.num_cand, g.k) == (rows, 8192, 2048)
        _check_rank_ranges(g, 32768)


def test_large_distribution():
    g = W.large(rows=8)
    assert g.num_cand == 8192 and g.k == 2048
    assert g.scores.min() >= -10 and g.scores.max() < 10
    _check_rank_ranges(g, 65536)


def test_tie_heavy_levels_and_empty_shards():
    g = W.tie_heavy(rows=16)
    real = g.ids != W.INT32_MAX
    assert set(np.unique(g.scores[real]).tolist()) <= set(W.TIE_LEVELS.tolist())
    for row in range(16):
        pads = np.nonzero(~real[row])[0]
        if row % 4 == 0:
            r = (row // 4) % 4
            assert np.array_equal(pads, np.arange(r * 2048, (r + 1) * 2048))
            assert np.all(np.isneginf(g.scores[row, pads]))
        else:
            assert pads.size == 0
    _check_rank_ranges(g, 32768)


def test_prefill_structure():
    sh = W.prefill(rows=32)
    assert sh.scores.shape == (4, 32, 2048) and sh.local_idx.shape == (4, 32, 2048)
    assert np.all((sh.local_idx >= 0) & (sh.local_idx < W.PREFILL_LOCAL_COLUMNS))
    for r in range(4):
        for t in range(32):
            assert len(np.unique(sh.local_idx[r, t])) == 2048
    assert np.all(sh.row_starts == sh.row_starts[0])
    assert np.all((sh.row_starts >= 0) & (sh.row_starts < W.PREFILL_ROW_START_SPAN))
    assert sh.rank_offsets.tolist() == [0, 135168, 270336, 405504]
