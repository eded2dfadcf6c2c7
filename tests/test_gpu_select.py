"""GPU parity of dcp_topk_select with the CPU oracle: bit-exact scores and ids.

Covers the named workloads at full size, the decode rows sweep, ragged sizes on
both load paths, the degenerate cases, heavy-tie trials, adversarial floats,
determinism and guard bands around the output.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, assert_select_parity, gpu_select, to_dev
from oracle import stable_topk as O
from stable_top_selection_amd import binding as B
from stable_top_selection_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()


@pytest.mark.parametrize("name", ["tiny", "decode", "large", "tie_heavy", "short_context"])
def test_workloads_full_size(name):
    g = getattr(W, name)()
    print(f"[select parity] {g.name} rows={g.rows} C={g.num_cand} k={g.k} digest={g.digest()}", flush=True)
    assert_select_parity(g.scores, g.ids, g.k, g.name, guard=2)


@pytest.mark.parametrize("rows", [1, 8, 32, 64])
def test_decode_rows_sweep(rows):
    g = W.decode(rows)
    assert_select_parity(g.scores, g.ids, g.k, g.name)


RAGGED = [
    # (rows, C, k, dist)
    (3, 1, 1, "normal"), (3, 2, 1, "normal"), (5, 3, 2, "uniform"), (4, 63, 7, "normal"),
    (4, 64, 63, "levels"), (4, 65, 64, "special"), (7, 255, 100, "normal"), (2, 256, 1, "uniform"),
    (3, 1000, 999, "normal"), (3, 1023, 500, "levels"), (3, 1024, 1023, "normal"), (3, 1025, 1, "special"),
    (5, 2047, 2046, "uniform"), (5, 2048, 2047, "normal"), (5, 2049, 1000, "levels"), (3, 3001, 1500, "const"),
    (4, 4095, 2048, "normal"), (4, 4096, 2048, "uniform"), (4, 4097, 2048, "levels"), (3, 6000, 5999, "special"),
    (3, 8191, 2048, "normal"), (3, 8193, 2048, "uniform"), (2, 12345, 4000, "levels"), (2, 16383, 2048, "normal"),
    (2, 16384, 2048, "uniform"), (2, 16384, 16383, "levels"), (2, 16384, 1, "normal"),
]


@pytest.mark.parametrize("rows,c,k,dist", RAGGED)
def test_ragged_sizes(rows, c, k, dist):
    g = W.random_gathered(rows, c, k, seed=1000 + c + k, dist=dist)
    assert_select_parity(g.scores, g.ids, k, g.name, guard=1)


@pytest.mark.parametrize("rows,c,k", [(3, 4096, 2048), (3, 8192, 2048), (2, 1000, 10)])
def test_eight_byte_load_path(rows, c, k):
    """A candidate buffer that is 8- but not 16-byte aligned takes the 8-byte loads."""
    g = W.random_gathered(rows, c, k, seed=77 + c, dist="normal")
    assert_select_parity(g.scores, g.ids, k, g.name, misalign=True)


@pytest.mark.parametrize("c,k", [(1, 1), (5, 9), (100, 100), (100, 2048), (8192, 8192), (8192, 9000)])
def test_k_at_least_num_cand_copies_and_pads(c, k):
    g = W.random_gathered(3, c, k, seed=c + k, dist="normal")
    assert_select_parity(g.scores, g.ids, k, g.name, guard=1)


def test_empty_rows_only_padding():
    out = torch.full((4, 5, 2), 7, dtype=torch.int32, device=DEV)
    B.select(torch.empty((4, 0, 2), dtype=torch.int32, device=DEV), 5, out=out)
    o = out.cpu().numpy()
    assert np.all(o[..., 0].view(np.uint32) == 0xFF800000) and np.all(o[..., 1] == 2**31 - 1)


def test_zero_rows_is_a_no_op():
    out = torch.empty((0, 4, 2), dtype=torch.int32, device=DEV)
    B.select(torch.empty((0, 16, 2), dtype=torch.int32, device=DEV), 4, out=out)


@pytest.mark.parametrize("dist,pad", [("levels", 0.3), ("const", 0.0), ("special", 0.5), ("normal", 0.9)])
def test_padding_and_full_duplicates(dist, pad):
    """Padding slots are identical (score, id) pairs; with repeated ids the
    boundary cuts through identical candidates and position decides."""
    g = W.random_gathered(8, 8192, 2048, seed=31, dist=dist, pad_frac=pad)
    assert_select_parity(g.scores, g.ids, g.k, g.name)
    g = W.random_gathered(8, 5000, 1234, seed=32, dist=dist, id_span=64, repeat_ids=True, pad_frac=pad)
    assert_select_parity(g.scores, g.ids, g.k, g.name)


def test_all_padding_and_all_tie_rows():
    c, k = 8192, 2048
    scores = np.full((4, c), -np.inf, np.float32)
    ids = np.full((4, c), 2**31 - 1, np.int32)
    scores[1] = 3.0
    ids[1] = np.random.default_rng(5).permutation(c).astype(np.int32)
    scores[2, :k] = 1.0  # exactly k real candidates, the rest padding
    ids[2, :k] = np.arange(k, dtype=np.int32)[::-1]
    scores[3, ::2] = 0.5  # every other slot real, ids all equal
    ids[3, ::2] = 9
    assert_select_parity(scores, ids, k, "all-padding / all-tie")


def test_heavy_tie_trials():
    """Many tie-heavy rows (every row ties at the threshold score), in the
    spirit of the repeated heavy-tie trials on PR #47348's review: 3 x 256 rows."""
    for seed in (11, 12, 13):
        g = W.tie_heavy(rows=256, seed=seed)
        assert_select_parity(g.scores, g.ids, g.k, f"tie_heavy seed {seed}")


def test_adversarial_floats():
    """NaNs of both signs and several payloads, +-0, +-inf, subnormals."""
    rng = np.random.default_rng(8)
    specials = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF, 0x7FFFFFFF, 0x80000000, 0x00000000,
                         0x7F800000, 0xFF800000, 0x00000001, 0x80000001, 0x3F800000, 0xBF800000], np.uint32)
    bits = rng.integers(0, 2**32, size=(16, 8192), dtype=np.uint64).astype(np.uint32)
    mask = rng.random(bits.shape) < 0.5
    bits = np.where(mask, specials[rng.integers(0, len(specials), size=bits.shape)], bits)
    ids = rng.integers(0, 50, size=bits.shape).astype(np.int32)
    for k in (1, 2048, 8191):
        assert_select_parity(bits.view(np.float32), ids, k, f"adversarial k={k}")


def test_negative_ids_compare_unsigned():
    """Outside the merge's id range: ids compare as uint32 through ~id."""
    scores = np.ones((2, 300), np.float32)
    ids = np.random.default_rng(3).integers(-2**31, 2**31 - 1, size=(2, 300), dtype=np.int64).astype(np.int32)
    assert_select_parity(scores, ids, 100, "negative ids")


def test_deterministic_repeats():
    g = W.tie_heavy(rows=64, seed=21)
    first = gpu_select(g.scores, g.ids, g.k)
    for _ in range(5):
        again = gpu_select(g.scores, g.ids, g.k)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])


def test_unsupported_and_invalid_arguments():
    cand = torch.zeros((2, 16385, 2), dtype=torch.int32, device=DEV)
    with pytest.raises(B.DcpTopkError) as e:
        B.select(cand, 10)
    assert e.value.status == B.EUNSUPPORTED
    cand = torch.zeros((2, 64, 2), dtype=torch.int32, device=DEV)
    with pytest.raises(B.DcpTopkError) as e:  # output aliasing the input
        B.select(cand, 64, out=cand)
    assert e.value.status == B.EINVAL


def test_graph_capture_replay_with_changing_inputs():
    """The select is a pure enqueue: capture once, replay on new inputs."""
    rows, c, k = 32, 8192, 2048
    static_in = torch.empty((rows, c, 2), dtype=torch.int32, device=DEV)
    static_out = torch.empty((rows, k, 2), dtype=torch.int32, device=DEV)
    g0 = W.random_gathered(rows, c, k, seed=100)
    static_in.copy_(to_dev(g0.interleaved()))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.select(static_in, k, out=static_out)  # warm up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.select(static_in, k, out=static_out)
    for seed in (101, 102, 103):
        g = W.random_gathered(rows, c, k, seed=seed, dist="levels" if seed % 2 else "normal")
        static_in.copy_(to_dev(g.interleaved()))
        graph.replay()
        torch.cuda.synchronize()
        want_b, want_i = gpu_select(g.scores, g.ids, k)  # eager run between replays
        o = static_out.cpu().numpy()
        assert np.array_equal(o[..., 0].view(np.uint32), want_b) and np.array_equal(o[..., 1], want_i)
        from oracle import stable_topk as O
        ob, oi = O.select(g.scores, g.ids, k)
        assert np.array_equal(want_b, ob.view(np.uint32)) and np.array_equal(want_i, oi)


def _sorted_within_ranks(g, descending=True):
    """Each rank slice of every row sorted by score: the first chunk the kernel
    sees is then far from a random sample of the row."""
    scores, ids = g.scores.copy(), g.ids.copy()
    lk = g.local_k
    for r in range(g.dcp):
        sl = slice(r * lk, (r + 1) * lk)
        order = np.argsort(scores[:, sl], axis=1, kind="stable")
        if descending:
            order = order[:, ::-1]
        scores[:, sl] = np.take_along_axis(scores[:, sl], order, axis=1)
        ids[:, sl] = np.take_along_axis(ids[:, sl], order, axis=1)
    return scores, ids


@pytest.mark.parametrize("descending", [True, False])
def test_rank_slices_sorted_by_score(descending):
    """Local top-K outputs are often sorted; the selection must not depend on
    the order of the candidates within a row."""
    for g in (W.decode(16), W.large(rows=32), W.tie_heavy(16)):
        s, i = _sorted_within_ranks(g, descending)
        assert_select_parity(s, i, g.k, f"{g.name} sorted desc={descending}")


def test_threshold_bin_sizes():
    """Threshold bins of about 1.5k items (more than one window segment holds)
    and of the whole row with distinct low bits (more than a list holds)."""
    rng = np.random.default_rng(71)
    rows, c, k = 6, 8192, 2048
    # ~1500 items share the threshold's top 11 bits: 1.5k values in [1, 1.0625)
    base = rng.standard_normal((rows, c)).astype(np.float32) * np.float32(0.01)
    near = (np.float32(1.0) + rng.random((rows, 1500), dtype=np.float32) * np.float32(0.0624)).astype(np.float32)
    s = np.concatenate([np.full((rows, 1000), 50.0, np.float32), near, base[:, : c - 2500]], axis=1)
    s = np.ascontiguousarray(np.take_along_axis(s, rng.permuted(np.tile(np.arange(c), (rows, 1)), axis=1), axis=1))
    ids = W.distinct_per_row(rng, rows, c, 4 * c)
    assert_select_parity(s, ids, k, "threshold bin ~1500")
    # every key shares its top 11 bits, the low bits differ
    s = (np.float32(1.0) + rng.random((rows, c), dtype=np.float32) * np.float32(0.0009)).astype(np.float32)
    assert_select_parity(s, ids, k, "one bin, distinct low bits")
    assert_select_parity(s, ids, 1, "one bin, k=1")


@pytest.mark.parametrize("rows,c,k", [(3, 2600, 1000), (3, 2560, 7), (2, 5000, 4999), (2, 9000, 3000)])
def test_rows_shorter_than_the_thread_slots(rows, c, k):
    """Rows whose last waves hold no candidate at all."""
    g = W.random_gathered(rows, c, k, seed=c, dist="uniform")
    assert_select_parity(g.scores, g.ids, k, g.name, guard=1)


@pytest.mark.parametrize("copies,same_id", [(1, False), (3, False), (7, True), (15, False), (20, False)])
def test_ties_at_the_threshold_in_a_small_sub_bin(copies, same_id):
    """A few copies of the K-th largest score (so the threshold's bin holds a
    handful of items that tie on the full key), optionally sharing one id (full
    duplicates straddling the boundary); 20 copies exceed the comparison path
    and take the histogram passes."""
    rng = np.random.default_rng(900 + copies)
    rows, c, k = 8, 8192, 2048
    s = rng.standard_normal((rows, c), dtype=np.float32)
    ids = W.distinct_per_row(rng, rows, c, 4 * c)
    for r in range(rows):
        kth = np.sort(s[r])[::-1][k - 1 + (r % 3) - 1]  # around the K-th largest
        below = np.nonzero(s[r] < kth)[0]
        at = rng.choice(below, copies, replace=False)
        s[r, at] = kth
        if same_id:
            tied = np.nonzero(s[r] == kth)[0]
            ids[r, tied[1:]] = ids[r, tied[0]]
    assert_select_parity(s, ids, k, f"{copies} copies of the threshold, shared id {same_id}")


def test_row_offsets_beyond_2_gib():
    """40960 rows of 8192 candidates (2.5 GiB of input, 640 MiB of output):
    row offsets past 2^31 bytes.  The rows repeat a seeded 64-row block, so
    every output row is checked against the oracle's result for its block row."""
    g = W.decode(64, seed=404)
    reps = 640
    block = to_dev(g.interleaved())
    cand = block.repeat(reps, 1, 1)
    assert cand.numel() * 4 > 2**31
    out = B.select(cand, g.k)
    torch.cuda.synchronize()
    want_s, want_i = O.select(g.scores, g.ids, g.k)
    want = np.stack([want_s.view(np.int32), want_i], axis=-1)
    o = out.view(reps, 64, g.k, 2)
    for r in (0, 1, reps // 2, reps - 1):
        assert np.array_equal(o[r].cpu().numpy(), want), f"block repeat {r} differs"
    del cand, out
    torch.cuda.empty_cache()


def test_max_rows():
    """DCP_TOPK_MAX_ROWS rows (4,194,303) of 3 candidates, k 2: the largest grid
    one select launch takes (256 threads per row, about 1.07e9 threads).  Every
    row is checked against the oracle, with score ties in a tenth of the rows;
    one row more is refused before any launch."""
    rows = B.MAX_ROWS
    rng = np.random.default_rng(4242)
    scores = rng.standard_normal((rows, 3), dtype=np.float32)
    tied = rng.random(rows) < 0.1
    scores[tied, 2] = scores[tied, 0]
    ids = rng.integers(0, 1 << 20, size=(rows, 3), dtype=np.int32)
    assert_select_parity(scores, ids, 2, "max rows")
    cand = torch.zeros((rows + 1, 3, 2), dtype=torch.int32, device=DEV)
    with pytest.raises(B.DcpTopkError) as e:
        B.select(cand, 2)
    assert e.value.status == B.EUNSUPPORTED
    del cand
    torch.cuda.empty_cache()


@pytest.mark.parametrize("c,k", [(1000, 300), (2048, 2047), (300, 1)])
def test_rows_of_one_repeated_candidate(c, k):
    """Every candidate identical (same score bits and id): the first k
    positions are taken, through the list path's all-duplicates branch."""
    rows = 3
    s = np.full((rows, c), 1.5, np.float32)
    s[1] = -np.inf
    s[2] = -0.0
    ids = np.full((rows, c), 77, np.int32)
    ids[1] = 2**31 - 1
    assert_select_parity(s, ids, k, f"one repeated candidate, C={c} k={k}")


@pytest.mark.parametrize("c,k,pad,misalign", [(3000, 2000, 0.5, False), (1200, 1000, 0.6, True),
                                              (8192, 2048, 0.78, False), (5000, 4990, 0.3, False)])
def test_padding_in_the_threshold_bin(c, k, pad, misalign):
    """Fewer real candidates than k, so the threshold falls among the padding
    keys, which pass 0 counts apart: padding slots plus real -inf scores with
    their own ids (ties on the -inf key, broken by id, then by position)."""
    g = W.random_gathered(4, c, k, seed=c + k, dist="normal", pad_frac=pad)
    s, ids = g.scores.copy(), g.ids.copy()
    rng = np.random.default_rng(c)
    real_inf = rng.random(s.shape) < 0.02
    s[real_inf] = -np.inf
    assert_select_parity(s, ids, k, f"padding threshold C={c} k={k} pad={pad}", misalign=misalign)


@pytest.mark.parametrize("k", [1, 2048, 5000])
def test_oversized_threshold_bin_common_bits(k):
    """Threshold bins of more than 2048 items (the register passes): bits that
    every item of the bin shares are fixed without a pass, so these rows hit
    each entry point of the key and id passes: identical keys with ids that
    differ only in their low 9 bits, only below bit 18 and in bit 31; keys
    that differ with ids that differ in 2 bits; padding mixed with real -inf
    scores."""
    rng = np.random.default_rng(4100 + k)
    rows, c = 6, 8192
    s = np.full((rows, c), 2.0, np.float32)
    ids = np.empty((rows, c), np.int32)
    ids[0] = rng.integers(0, 512, size=c)
    ids[1] = 0x12340000 + rng.integers(0, 1 << 18, size=c)
    s[2] = (np.float32(1.0) + rng.random(c, dtype=np.float32) * np.float32(0.0009)).astype(np.float32)
    ids[2] = 5 + rng.integers(0, 4, size=c)
    s[3] = -np.inf
    ids[3] = np.where(rng.random(c) < 0.5, 2**31 - 1, rng.permutation(c)).astype(np.int32)
    s[4] = -0.0
    ids[4] = 42
    ids[4, rng.choice(c, 100, replace=False)] = -42
    s[5] = 2.0
    ids[5] = rng.permutation(c)
    assert_select_parity(s, ids, k, f"oversized threshold bins k={k}")
