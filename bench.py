#!/usr/bin/env python3
"""Benchmark of the stable DCP top-K select on one MI355X.

Headline (one JSON line on stdout): ``dcp_topk_select`` on the large workload,
256 rows x 8192 candidates (DCP 4 x local K 2048), K 2048, scores U(-10,10).
One step = one select launch over the whole batch.  Algorithmic bytes per
launch = rows*C*8 read + rows*K*8 written = 20,971,520.

Timing follows the pages' selector microbenchmark (PR #47348, Benchmarks:
median over 7 trials of 200 launches, warm-up excluded).  The launches of a
trial are captured once in a HIP graph and replayed, so the per-launch time is
the GPU's and not the host's launch rate; HIP events on the replay stream
bracket every trial.  A trial is at least 200 launches whatever ``--steps``
asks (more when the input pool is larger), so that the graph's own launch
cost is spread as in the pages' method; the JSON's ``steps`` is the number of
launches actually timed (trials x launches per trial).  Inputs rotate through a pool larger than twice the
MI355X's Infinity Cache plus L2 (2 x (256 + 32) MiB), so every launch reads its
candidates from HBM ("cold").  Warm-cache numbers (one buffer reused) are
reported separately and labelled.

Other lines of the same JSON object: the decode rows sweep and the tie-heavy
workload as latencies, the chunked prefill merge (T = 8192) as a whole-driver
time, the fused merge (no gathered buffer) on the large shape and on the
prefill workload, the local top-K (2048 of 4096 columns), the CPU oracle timed
on the host (``cpu_baseline``), and the roofline of the select kernel.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "select µs/launch + candidates/s and % peak HBM BW (rows=256, 8192 cand, K=2048)"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD published peak
MIB = 1 << 20
COLD_POOL_BYTES = 2 * (256 + 32) * MIB  # 2 x (Infinity Cache + 8 x 4 MiB L2)
MIN_LAUNCHES = 200  # launches per timed trial, at least (PR #47348, Benchmarks: 7 x 200)
CAND_BYTES = 8
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "select_large_rows256_traffic.json")
SELECT_SOURCE = os.path.join(ROOT, "stable_top_selection_amd", "csrc", "select.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200,
                   help="select launches per timed trial (at least 200 are timed, a whole number of pool passes)")
    p.add_argument("--warmup", type=int, default=20, help="untimed launches before timing")
    p.add_argument("--trials", type=int, default=7)
    p.add_argument("--configs", default="large,large_warm,large_eager,decode,pages,split,tie_heavy,short_context,prefill,fused,local",
                   help="comma list of large_warm, large_eager, decode, pages, split, tie_heavy, short_context, prefill, fused, "
                        "local; the cold large headline always runs (--configs large runs it alone, as profiled)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle work to time")
    p.add_argument("--pmc", action="store_true",
                   help="counter-collection mode: a 512 MiB torch copy (calibration) then cold select launches, "
                        "no timing and no JSON")
    return p.parse_args()


def select_bytes(rows, c, k):
    return rows * c * CAND_BYTES + rows * k * CAND_BYTES


class Runner:
    """Raw C-ABI launches with precomputed pointers (no per-call Python checks)."""

    def __init__(self):
        import torch

        from stable_top_selection_amd import binding as B

        self.torch = torch
        self.B = B
        self.lib = B.load_library()
        self.dev = torch.device("cuda:0")

    def select(self, cand_ptr, rows, c, k, out_ptr, stream_ptr):
        st = self.lib.dcp_topk_select(cand_ptr, rows, c, k, out_ptr, stream_ptr)
        if st != 0:
            raise RuntimeError(f"dcp_topk_select: {self.B.status_string(st)}")

    def stream_ptr(self):
        return self.torch.cuda.current_stream().cuda_stream

    def graph_of(self, fns):
        """Capture fns (each takes a stream pointer) into one HIP graph."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fns[0](self.stream_ptr())  # first launch outside capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sp = self.stream_ptr()
            for f in fns:
                f(sp)
        return g

    def time_graph(self, g, trials):
        """Milliseconds of each replay, bracketed by events on the replay stream."""
        torch = self.torch
        g.replay()
        torch.cuda.synchronize()
        out = []
        for _ in range(trials):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            e1.synchronize()
            out.append(e0.elapsed_time(e1))
        return out


def make_pool(run, inter, k, pool_bytes):
    """Copies of one input (rows, C, 2) int32 spread over >= pool_bytes, with
    one output per copy.  Returns (list of (cand_ptr, out_ptr), tensors)."""
    torch = run.torch
    rows, c, _ = inter.shape
    per = select_bytes(rows, c, k)
    n = max(1, -(-pool_bytes // per))
    src = torch.from_numpy(inter).to(run.dev)
    cands = torch.empty((n, rows, c, 2), dtype=torch.int32, device=run.dev)
    cands.copy_(src.unsqueeze(0).expand(n, rows, c, 2))
    outs = torch.empty((n, rows, k, 2), dtype=torch.int32, device=run.dev)
    ptrs = [(cands[i].data_ptr(), outs[i].data_ptr()) for i in range(n)]
    return ptrs, (src, cands, outs)


def check_pool_outputs(run, tensors, gathered, k, sample):
    """Bit-exact check of sampled pool outputs against the CPU oracle."""
    import numpy as np

    from oracle import stable_topk as oracle

    _, cands, outs = tensors
    want_s, want_i = oracle.select(gathered.scores, gathered.ids, k)
    idx = sorted(set([0, outs.shape[0] - 1] + list(range(0, outs.shape[0], max(1, outs.shape[0] // sample)))))
    for i in idx:
        o = outs[i].cpu().numpy()
        if not (np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)) and np.array_equal(o[..., 1], want_i)):
            raise AssertionError(f"bench output {i} differs from the oracle ({gathered.name})")
    return len(idx)


def launches_per_trial(steps, pool):
    """At least MIN_LAUNCHES and ``steps`` launches, a whole number of passes
    over an input pool of ``pool`` buffers."""
    want = max(MIN_LAUNCHES, steps)
    return -(-want // pool) * pool


def bench_select(run, g, steps, warmup, trials, cold=True, select=None):
    """Median per-launch microseconds of a graph of launches rotating over a
    cold pool (``select``, with run.select's arguments, replaces the launch)."""
    select = select or run.select
    inter = g.interleaved()
    pool_bytes = COLD_POOL_BYTES if cold else 0
    ptrs, tensors = make_pool(run, inter, g.k, pool_bytes)
    n = len(ptrs)
    launches = launches_per_trial(steps, n)
    rows, c, k = g.rows, g.num_cand, g.k

    def fn(i):
        cp, op = ptrs[i % n]
        return lambda sp: select(cp, rows, c, k, op, sp)

    for i in range(warmup):
        fn(i)(run.stream_ptr())
    run.torch.cuda.synchronize()
    graph = run.graph_of([fn(i) for i in range(launches)])
    ms = run.time_graph(graph, trials)
    checked = check_pool_outputs(run, tensors, g, k, sample=4)
    us = [1e3 * m / launches for m in ms]
    del graph, tensors
    run.torch.cuda.empty_cache()
    med = statistics.median(us)
    gbps = select_bytes(rows, c, k) / (med * 1e-6) / 1e9
    return {"us_per_launch": med, "us_trials": [round(x, 4) for x in us], "launches": launches,
            "pool_buffers": n, "outputs_checked": checked, "candidates_per_s": rows * c / (med * 1e-6),
            "GBps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_HBM_GBS, 4)}


def bench_split(run, steps, warmup, trials, decode=None):
    """The split-row select (each row over 2, 4 or 8 workgroups) on the decode
    rows, cold, beside the one-workgroup select's cold latency on the same
    inputs."""
    from stable_top_selection_amd import workloads as W
    torch, lib = run.torch, run.lib
    out = {}
    for rows in (1, 8, 16, 32, 64):
        g = W.decode(rows)
        line = {"one_workgroup_cold_us": decode[f"rows{rows}"]["cold_us"] if decode else None}
        for parts in (2, 4, 8):
            ws = run.B.select_split_workspace(rows, g.num_cand, parts, run.dev)

            def split(cp, r, c, k, op, sp, ws=ws, parts=parts):
                st = lib.dcp_topk_select_split(run.B._p(cp), r, c, k, parts, run.B._p(ws.data_ptr()), ws.numel(),
                                               run.B._p(op), sp)
                if st != 0:
                    raise run.B.DcpTopkError("dcp_topk_select_split", st)

            res = bench_select(run, g, steps, warmup, trials, cold=True, select=split)
            line[f"parts{parts}_cold_us"] = round(res["us_per_launch"], 3)
            del ws
        out[f"rows{rows}"] = line
        log(f"[split rows={rows}] {line}")
    torch.cuda.empty_cache()
    return out


# The pages' selector table (PR #47348, Benchmarks: median us of 7 x 200
# launches; hardware, K and score distributions not stated): (rows, candidates,
# distribution) -> us of the PR's selector.  Context only.
PAGES_SELECTOR_US = [((16, 4096, "random"), 6.721), ((16, 8192, "random"), 11.478),
                     ((16, 16384, "random"), 20.684), ((64, 8192, "random"), 11.696),
                     ((256, 8192, "random"), 15.459), ((16, 8192, "tie-heavy"), 20.396)]


def bench_pages_table(run, steps, warmup, trials):
    """Every case of the pages' selector table with this select, cold pools,
    K 2048: "random" rows of 8192 are the decode workload (N(0,1)) at 16 and
    64 rows and the large workload (U(-10,10)) at 256; 4096 and 16384 use
    N(0,1) scores with distinct ids; "tie-heavy" is the tie-heavy workload."""
    from stable_top_selection_amd import workloads as W
    out = []
    for (rows, c, dist), pages_us in PAGES_SELECTOR_US:
        if dist == "tie-heavy":
            g = W.tie_heavy(rows=rows)
        elif c == 8192:
            g = W.large() if rows == 256 else W.decode(rows)
        else:
            g = W.random_gathered(rows, c, 2048, seed=4700 + c, dist="normal")
        res = bench_select(run, g, steps, warmup, trials, cold=True)
        us = res["us_per_launch"]
        out.append({"rows": rows, "candidates": c, "distribution": dist, "workload": g.name, "k": g.k,
                    "cold_us": round(us, 3), "pages_us": pages_us, "pages_over_this": round(pages_us / us, 2)})
        log(f"[pages table] rows={rows} C={c} {dist}: {us:.3f} us (pages {pages_us} us)")
    return out


def bench_eager(run, g, steps, trials):
    """Same launches without a graph (host launch rate included), cold pool."""
    ptrs, tensors = make_pool(run, g.interleaved(), g.k, COLD_POOL_BYTES)
    torch = run.torch
    n = len(ptrs)
    res = []
    sp = run.stream_ptr()
    for _ in range(trials):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            cp, op = ptrs[i % n]
            run.select(cp, g.rows, g.num_cand, g.k, op, sp)
        e1.record()
        e1.synchronize()
        res.append(1e3 * e0.elapsed_time(e1) / steps)
    del tensors
    return statistics.median(res)


PREFILL_REPEATS = 5  # whole merges (or pack / select passes) per graph replay


def bench_prefill(run, trials):
    """Whole chunked merge at T = 8192 (8 chunks of 1024 rows), PREFILL_REPEATS
    merges per graph replay so that the replay's own start-up is spread as in
    the select timing, and the select and pack launches of the same chunks on
    their own (the same number of passes per replay)."""
    import ctypes

    import numpy as np

    from oracle import stable_topk as oracle
    from stable_top_selection_amd import workloads as W

    torch = run.torch
    sh = W.prefill()
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(run.dev)  # noqa: E731
    sc = [to(sh.scores[r]) for r in range(sh.dcp)]
    ix = [to(sh.local_idx[r]) for r in range(sh.dcp)]
    rs = [to(sh.row_starts[r]) for r in range(sh.dcp)]
    offs = [int(x) for x in sh.rank_offsets]
    T, dcp, lk, k = sh.rows, sh.dcp, sh.local_k, sh.k
    need = run.B.merge_workspace_bytes(T, dcp, lk)
    ws = torch.empty(need, dtype=torch.uint8, device=run.dev)
    out = torch.empty((T, k, 2), dtype=torch.int32, device=run.dev)
    arr = ctypes.c_void_p * dcp
    sp_, ip_, rp_ = arr(*[t.data_ptr() for t in sc]), arr(*[t.data_ptr() for t in ix]), arr(*[t.data_ptr() for t in rs])
    of_ = (ctypes.c_int32 * dcp)(*offs)
    cast = lambda x: ctypes.cast(x, ctypes.c_void_p)  # noqa: E731

    def merge(stream_ptr):
        st = run.lib.dcp_topk_merge_chunked(cast(sp_), cast(ip_), cast(rp_), cast(of_), dcp, T, lk, k,
                                            ws.data_ptr(), need, out.data_ptr(), stream_ptr)
        if st != 0:
            raise RuntimeError(run.B.status_string(st))

    graph = run.graph_of([merge] * PREFILL_REPEATS)
    ms = [m / PREFILL_REPEATS for m in run.time_graph(graph, trials)]
    # sampled rows against the oracle (the oracle on all 8192 rows takes ~10 s)
    rows = np.unique(np.concatenate([np.arange(0, T, 97), [1023, 1024, 4095, 4096, T - 1]]))
    want_s, want_i = oracle.merge(sh.scores[:, rows], sh.local_idx[:, rows], sh.row_starts[:, rows], sh.rank_offsets, k)
    o = out.cpu().numpy()[rows]
    if not (np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)) and np.array_equal(o[..., 1], want_i)):
        raise AssertionError("prefill merge differs from the oracle on sampled rows")
    # select alone on the 8 chunk-sized gathered buffers the merge builds (the
    # workspace is MALL-resident, as it is when the merge's select reads what
    # its pack just wrote)
    gathered = ws.view(torch.int32).view(min(T, 1024), dcp * lk, 2)
    chunk_outs = [out[c0:c0 + 1024] for c0 in range(0, T, 1024)]
    sel = [lambda spp, o_=o_: run.select(gathered.data_ptr(), 1024, dcp * lk, k, o_.data_ptr(), spp)
           for o_ in chunk_outs]
    g2 = run.graph_of(sel * PREFILL_REPEATS)
    ms_sel = [m / PREFILL_REPEATS for m in run.time_graph(g2, trials)]
    # pack alone: dcp_topk_pack of every rank of every chunk into the
    # workspace (one rank per launch; the chunked driver packs all ranks of a
    # chunk in one launch of the same kernel)
    ws_ptr = ws.data_ptr()

    def pack_launch(c0, r):
        n = min(1024, T - c0)

        def f(spp):
            st = run.lib.dcp_topk_pack(sc[r].data_ptr() + 4 * c0 * lk, ix[r].data_ptr() + 4 * c0 * lk, lk,
                                       rs[r].data_ptr() + 4 * c0, offs[r], n, lk, ws_ptr + 8 * r * lk, dcp * lk, spp)
            if st != 0:
                raise RuntimeError(run.B.status_string(st))
        return f

    g3 = run.graph_of([pack_launch(c0, r) for c0 in range(0, T, 1024) for r in range(dcp)] * PREFILL_REPEATS)
    ms_pack = [m / PREFILL_REPEATS for m in run.time_graph(g3, trials)]
    merge_ms = statistics.median(ms)
    sel_ms = statistics.median(ms_sel)
    pack_ms = statistics.median(ms_pack)
    chunks = -(-T // 1024)
    sel_bytes = chunks * select_bytes(1024, dcp * lk, k)
    pack_bytes = T * dcp * lk * (4 + 4 + 8) + dcp * T * 4
    gb = lambda b, t_ms: b / (t_ms * 1e-3) / 1e9  # noqa: E731
    return {"workload": f"prefill chunked: T={T}, DCP {dcp} x local K {lk}, K {k}, 1024-row chunks",
            "merges_per_replay": PREFILL_REPEATS,
            "merge_ms": round(merge_ms, 4), "merge_trials_ms": [round(x, 4) for x in ms],
            "merge_GBps": round(gb(sel_bytes + pack_bytes, merge_ms), 1),
            "merge_candidates_per_s": round(T * dcp * lk / (merge_ms * 1e-3)),
            "select_only_ms": round(sel_ms, 4), "per_chunk_select_us": round(1e3 * sel_ms / chunks, 2),
            "select_GBps_MALL_resident_workspace": round(gb(sel_bytes, sel_ms), 1),
            "select_frac_of_peak": round(gb(sel_bytes, sel_ms) / PEAK_HBM_GBS, 4),
            "pack_only_ms": round(pack_ms, 4), "pack_launches": chunks * dcp,
            "pack_GBps": round(gb(pack_bytes, pack_ms), 1),
            "pack_frac_of_peak": round(gb(pack_bytes, pack_ms) / PEAK_HBM_GBS, 4),
            "pack_algorithmic_bytes": pack_bytes,
            "rows_checked": int(len(rows))}


class RankPtrs:
    """Host arrays of one launch's per-rank device pointers (kept alive)."""

    def __init__(self, scores, idx, starts, offsets):
        import ctypes

        n = len(scores)
        arr = ctypes.c_void_p * n
        self.s = arr(*[t.data_ptr() for t in scores])
        self.i = arr(*[t.data_ptr() for t in idx])
        self.r = arr(*[t.data_ptr() for t in starts])
        self.o = (ctypes.c_int32 * n)(*[int(x) for x in offsets])
        self.args = [ctypes.cast(x, ctypes.c_void_p) for x in (self.s, self.i, self.r, self.o)]


def bench_fused(run, steps, warmup, trials):
    """The fused merge (select straight from the ranks' local arrays):
    (1) on the large shape (256 rows, DCP 4 x local K 2048, K 2048), HBM-cold
    pool, per launch; (2) on the prefill workload, all T = 8192 rows in one
    launch, against the chunked merge of the same inputs."""
    import numpy as np

    from oracle import stable_topk as oracle
    from stable_top_selection_amd import workloads as W

    torch = run.torch
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(run.dev)  # noqa: E731
    res = {}

    sh = W.fused()
    dcp, rows, lk, k = sh.dcp, sh.rows, sh.local_k, sh.k
    per = select_bytes(rows, dcp * lk, k)
    n = max(1, -(-COLD_POOL_BYTES // per))
    sc = to(sh.scores).unsqueeze(0).repeat(n, 1, 1, 1)
    ix = to(sh.local_idx).unsqueeze(0).repeat(n, 1, 1, 1)
    rs = [to(sh.row_starts[r]) for r in range(dcp)]
    outs = torch.empty((n, rows, k, 2), dtype=torch.int32, device=run.dev)
    ptrs = [RankPtrs([sc[i, r] for r in range(dcp)], [ix[i, r] for r in range(dcp)], rs, sh.rank_offsets)
            for i in range(n)]

    def launch(i):
        def f(sp):
            st = run.lib.dcp_topk_merge_fused(*ptrs[i % n].args, dcp, rows, lk, k, outs[i % n].data_ptr(), sp)
            if st != 0:
                raise RuntimeError(run.B.status_string(st))
        return f

    for i in range(warmup):
        launch(i)(run.stream_ptr())
    launches = launches_per_trial(steps, n)
    graph = run.graph_of([launch(i) for i in range(launches)])
    ms = run.time_graph(graph, trials)
    us = statistics.median([1e3 * m / launches for m in ms])
    want_s, want_i = oracle.merge(sh.scores, sh.local_idx, sh.row_starts, sh.rank_offsets, k)
    for i in (0, n - 1):
        o = outs[i].cpu().numpy()
        if not (np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)) and np.array_equal(o[..., 1], want_i)):
            raise AssertionError("fused merge output differs from the oracle")
    fused_bytes = per + dcp * rows * 4
    res["large_shape_cold"] = {"workload": f"{sh.name}: {rows} rows, DCP {dcp} x local K {lk}, K {k}",
                               "us_per_launch": round(us, 3), "pool_buffers": n, "launches": launches,
                               "GBps": round(fused_bytes / (us * 1e-6) / 1e9, 1),
                               "algorithmic_bytes_per_launch": fused_bytes}
    del graph, sc, ix, outs, ptrs
    torch.cuda.empty_cache()

    sh = W.prefill()
    dcp, T, lk, k = sh.dcp, sh.rows, sh.local_k, sh.k
    sc = [to(sh.scores[r]) for r in range(dcp)]
    ix = [to(sh.local_idx[r]) for r in range(dcp)]
    rs = [to(sh.row_starts[r]) for r in range(dcp)]
    out = torch.empty((T, k, 2), dtype=torch.int32, device=run.dev)
    rp = RankPtrs(sc, ix, rs, sh.rank_offsets)

    def fused(sp):
        st = run.lib.dcp_topk_merge_fused(*rp.args, dcp, T, lk, k, out.data_ptr(), sp)
        if st != 0:
            raise RuntimeError(run.B.status_string(st))

    graph = run.graph_of([fused] * PREFILL_REPEATS)
    ms = statistics.median([m / PREFILL_REPEATS for m in run.time_graph(graph, trials)])
    rows = np.unique(np.concatenate([np.arange(0, T, 97), [1023, 1024, 4095, 4096, T - 1]]))
    want_s, want_i = oracle.merge(sh.scores[:, rows], sh.local_idx[:, rows], sh.row_starts[:, rows],
                                  sh.rank_offsets, k)
    o = out.cpu().numpy()[rows]
    if not (np.array_equal(o[..., 0].view(np.uint32), want_s.view(np.uint32)) and np.array_equal(o[..., 1], want_i)):
        raise AssertionError("fused prefill merge differs from the oracle on sampled rows")
    pre_bytes = T * dcp * lk * 8 + T * k * 8 + dcp * T * 4
    res["prefill_one_launch"] = {"workload": f"prefill: T={T}, DCP {dcp} x local K {lk}, K {k}, one launch "
                                             f"({PREFILL_REPEATS} per graph replay)",
                                 "ms": round(ms, 4), "GBps": round(pre_bytes / (ms * 1e-3) / 1e9, 1),
                                 "rows_checked": int(len(rows))}
    return res


def bench_local(run, steps, warmup, trials):
    """Local top-K, 2048 of 4096 columns per row: rows 64 (the largest decode
    row count measured on PR #50009) and 256, HBM-cold pools, rows 64 warm,
    and with per-row lengths (rows 64 and 256; 2048 rows of 8192 columns,
    8 rows per CU, where the partial-row kernels' occupancy shows)."""
    import numpy as np

    from oracle import stable_topk as oracle
    from stable_top_selection_amd import workloads as W

    torch = run.torch
    res = {}
    for rows, cold, lengths, ncols in ((64, True, False, 4096), (64, False, False, 4096), (256, True, False, 4096),
                                       (64, True, True, 4096), (256, True, True, 4096), (2048, True, True, 8192)):
        d = W.local(rows=rows, num_cols=ncols, with_lengths=lengths)
        cols, k = d.num_cols, d.k
        per = rows * cols * 4 + rows * k * 8
        n = max(1, -(-COLD_POOL_BYTES // per)) if cold else 1
        src = torch.from_numpy(d.scores).to(run.dev).unsqueeze(0).repeat(n, 1, 1)
        os_ = torch.empty((n, rows, k), dtype=torch.float32, device=run.dev)
        oi = torch.empty((n, rows, k), dtype=torch.int32, device=run.dev)
        lens = torch.from_numpy(d.lengths).to(run.dev) if lengths else None
        lens_ptr = lens.data_ptr() if lengths else None

        def launch(i):
            def f(sp):
                st = run.lib.dcp_topk_local(src[i % n].data_ptr(), cols, lens_ptr, rows, cols, k,
                                            os_[i % n].data_ptr(), oi[i % n].data_ptr(), k, sp)
                if st != 0:
                    raise RuntimeError(run.B.status_string(st))
            return f

        for i in range(warmup):
            launch(i)(run.stream_ptr())
        launches = launches_per_trial(steps, n)
        graph = run.graph_of([launch(i) for i in range(launches)])
        us = statistics.median([1e3 * m / launches for m in run.time_graph(graph, trials)])
        ws, wi = oracle.local_topk(d.scores, k, d.lengths)
        for i in (0, n - 1):
            if not (np.array_equal(os_[i].cpu().numpy().view(np.uint32), ws.view(np.uint32))
                    and np.array_equal(oi[i].cpu().numpy(), wi)):
                raise AssertionError(f"local top-K output differs from the oracle ({d.name})")
        res[f"rows{rows}{'' if ncols == 4096 else f'_cols{ncols}'}_{'cold' if cold else 'warm'}"
            f"{'_lengths' if lengths else ''}"] = {
            "us_per_launch": round(us, 3), "GBps": round(per / (us * 1e-6) / 1e9, 1), "pool_buffers": n,
            "algorithmic_bytes_per_launch": per}
        del graph, src, os_, oi, lens
        torch.cuda.empty_cache()
    res["workload"] = ("local top-K: 4096 fp32 columns per row (8192 where named), k 2048, scores N(0,1); "
                       "'_lengths' lines take per-row lengths U[0, columns] (the partial-row kernels)")
    return res


# Arrays the CPU-baseline workers read.  The pool forks before this process
# touches the GPU, so the workers share them copy-on-write and never hold any
# GPU state.
_CPU = {}


def _cpu_select_rows(bounds):
    """One worker's share of a batch: the oracle on rows [lo, hi)."""
    from oracle import stable_topk as oracle

    lo, hi = bounds
    s, i = oracle.select(_CPU["scores"][lo:hi], _CPU["ids"][lo:hi], _CPU["k"])
    return int(i[:, :4].astype("int64").sum())  # a checksum: the results stay in the worker


def _cpu_merge_rows(bounds):
    """One worker's share of the prefill merge: pack + select of rows [lo, hi)."""
    from oracle import stable_topk as oracle

    lo, hi = bounds
    sh = _CPU["shards"]
    s, i = oracle.merge(sh.scores[:, lo:hi], sh.local_idx[:, lo:hi], sh.row_starts[:, lo:hi], sh.rank_offsets,
                        sh.k)
    return int(i[:, :4].astype("int64").sum())


def _blocks(rows, parts):
    step = -(-rows // parts)
    return [(lo, min(rows, lo + step)) for lo in range(0, rows, step)]


def _timed_runs(fn, seconds, min_runs=3):
    times = []
    t_end = time.perf_counter() + seconds
    while len(times) < min_runs or time.perf_counter() < t_end:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return times


def cpu_baselines(seconds):
    """The CPU oracle (numpy, one sort per row block) timed on this host: on
    every CPU of the process's affinity mask (a forked process pool over row
    blocks) and on one core, for the large batch; the pool also on the decode
    and tie-heavy batches and on the whole prefill merge (pack + select of
    T = 8192 rows).  Must run before anything touches the GPU."""
    import multiprocessing

    from oracle import stable_topk as oracle
    from stable_top_selection_amd import workloads as W

    cores = len(os.sched_getaffinity(0))
    out = {"cores_in_affinity_mask": cores}
    g = W.large()
    ctx = multiprocessing.get_context("fork")
    res = {}  # the pool forks at creation: one pool per batch, created after its arrays are set
    for name, gb, secs in (("large", g, seconds), ("decode_rows16", W.decode(16), min(2.0, seconds)),
                           ("tie_heavy", W.tie_heavy(), min(2.0, seconds))):
        _CPU.update(scores=gb.scores, ids=gb.ids, k=gb.k)
        with ctx.Pool(cores) as pool:
            blocks = _blocks(gb.rows, cores)
            pool.map(_cpu_select_rows, blocks, chunksize=1)  # warm the workers
            times = _timed_runs(lambda: pool.map(_cpu_select_rows, blocks, chunksize=1), secs)
        t = statistics.median(times)
        res[name] = {"candidates_per_s": gb.rows * gb.num_cand / t, "ms_per_batch": round(1e3 * t, 3),
                     "runs": len(times), "batch": f"{gb.rows} x {gb.num_cand}, K {gb.k}"}
        log(f"[cpu oracle, {cores} cores] {name}: {t * 1e3:.1f} ms per batch")
    times = _timed_runs(lambda: oracle.select(g.scores, g.ids, g.k), min(3.0, seconds))
    t1 = statistics.median(times)
    res["large_one_core"] = {"candidates_per_s": g.rows * g.num_cand / t1, "ms_per_batch": round(1e3 * t1, 3),
                             "runs": len(times), "cores": 1}
    log(f"[cpu oracle, 1 core] large: {t1 * 1e3:.1f} ms per batch")
    sh = W.prefill()
    _CPU.update(shards=sh)
    with ctx.Pool(cores) as pool:
        blocks = _blocks(sh.rows, 4 * cores)
        times = _timed_runs(lambda: pool.map(_cpu_merge_rows, blocks, chunksize=1), 0.0, min_runs=2)
    tm = statistics.median(times)
    res["prefill_merge_T8192"] = {"candidates_per_s": sh.rows * sh.dcp * sh.local_k / tm, "ms": round(1e3 * tm, 1),
                                  "runs": len(times),
                                  "work": f"pack + select of T={sh.rows} rows, DCP {sh.dcp} x local K {sh.local_k}, "
                                          f"K {sh.k}"}
    log(f"[cpu oracle, {cores} cores] prefill merge T={sh.rows}: {tm * 1e3:.0f} ms")
    _CPU.clear()
    big = res["large"]
    head = {"value": big["candidates_per_s"], "unit": "candidates/s", "cores": cores, "kind": "oracle",
            "sample": f"the full {g.name} batch ({g.rows} x {g.num_cand}, K {g.k}) through the numpy oracle, "
                      f"rows split over a pool of {cores} forked processes, median of {big['runs']} runs "
                      f"({big['ms_per_batch']:.1f} ms per batch)"}
    out.update(res)
    return head, out


def traffic_record(launch_us):
    """HBM traffic per launch from the committed counter summary, only if it
    was taken on the select kernel source as it is now."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    with open(SELECT_SOURCE, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if rec.get("select_source_sha256") != digest:
        return None
    return rec.get("bytes_per_launch")


def pmc_mode(run):
    """Fixed short sequence for rocprofv3 --pmc: a known-size copy, then cold selects."""
    from stable_top_selection_amd import workloads as W

    torch = run.torch
    n = 512 * MIB // 4
    a = torch.ones(n, dtype=torch.int32, device=run.dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    g = W.large()
    ptrs, tensors = make_pool(run, g.interleaved(), g.k, COLD_POOL_BYTES)
    sp = run.stream_ptr()
    for i in range(64):
        cp, op = ptrs[i % len(ptrs)]
        run.select(cp, g.rows, g.num_cand, g.k, op, sp)
    torch.cuda.synchronize()
    log(f"pmc mode: 3 copies of {512} MiB, then 64 cold select launches ({len(ptrs)} pool buffers)")


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the select path is not sharded across GPUs "
              "(each DCP rank runs the same select on its own gathered buffer); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    from stable_top_selection_amd import workloads as W

    # the CPU oracle first: its process pool forks before this process
    # touches the GPU
    cpu, cpu_extra = (None, None) if (args.no_cpu or args.pmc) else cpu_baselines(args.cpu_seconds)
    run = Runner()
    if args.pmc:
        pmc_mode(run)
        return
    configs = [c.strip() for c in args.configs.split(",") if c.strip()]
    props = run.torch.cuda.get_device_properties(run.dev)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")

    g = W.large()
    log(f"[large] rows={g.rows} C={g.num_cand} k={g.k} digest={g.digest()}")
    res = bench_select(run, g, args.steps, args.warmup, args.trials, cold=True)
    us = res["us_per_launch"]
    per_launch_bytes = select_bytes(g.rows, g.num_cand, g.k)
    gbs = per_launch_bytes / (us * 1e-6) / 1e9
    log(f"[large] cold {us:.3f} us/launch, {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of peak)")
    extra = {"large_cold": res}
    if "large_warm" in configs:
        warm = bench_select(run, g, args.steps, args.warmup, args.trials, cold=False)
        extra["large_warm_L2_MALL_not_HBM"] = warm
        log(f"[large] warm (one buffer, cache-resident) {warm['us_per_launch']:.3f} us/launch")
    if "large_eager" in configs:
        eager = bench_eager(run, g, args.steps, args.trials)
        extra["large_eager_cold_us_per_launch"] = round(eager, 4)
        log(f"[large] eager launches (host launch rate included) {eager:.3f} us/launch")
    if "decode" in configs:
        sweep = {}
        for rows in (1, 8, 16, 32, 64):
            gd = W.decode(rows)
            cold = bench_select(run, gd, args.steps, args.warmup, args.trials, cold=True)
            hot = bench_select(run, gd, args.steps, args.warmup, args.trials, cold=False)
            sweep[f"rows{rows}"] = {"cold_us": round(cold["us_per_launch"], 3), "warm_us": round(hot["us_per_launch"], 3),
                                    "cold_candidates_per_s": round(cold["candidates_per_s"]), "cold_GBps": cold["GBps"],
                                    "cold_frac_of_peak": cold["frac_of_peak"]}
            log(f"[decode rows={rows}] cold {cold['us_per_launch']:.3f} us, warm {hot['us_per_launch']:.3f} us")
        extra["decode_latency_us"] = sweep
    if "pages" in configs:
        extra["pages_selector_table"] = bench_pages_table(run, args.steps, args.warmup, args.trials)
    if "split" in configs:
        extra["split_rows_latency_us"] = bench_split(run, args.steps, args.warmup, args.trials,
                                                     extra.get("decode_latency_us"))
    if "tie_heavy" in configs:
        gt = W.tie_heavy()
        cold = bench_select(run, gt, args.steps, args.warmup, args.trials, cold=True)
        hot = bench_select(run, gt, args.steps, args.warmup, args.trials, cold=False)
        extra["tie_heavy_latency_us"] = {"rows": gt.rows, "cold_us": round(cold["us_per_launch"], 3),
                                         "warm_us": round(hot["us_per_launch"], 3),
                                         "cold_candidates_per_s": round(cold["candidates_per_s"]),
                                         "cold_GBps": cold["GBps"], "cold_frac_of_peak": cold["frac_of_peak"]}
        log(f"[tie_heavy] cold {cold['us_per_launch']:.3f} us, warm {hot['us_per_launch']:.3f} us")
    if "short_context" in configs:
        gs = W.short_context()
        cold = bench_select(run, gs, args.steps, args.warmup, args.trials, cold=True)
        hot = bench_select(run, gs, args.steps, args.warmup, args.trials, cold=False)
        extra["short_context_latency_us"] = {"rows": gs.rows, "cold_us": round(cold["us_per_launch"], 3),
                                             "warm_us": round(hot["us_per_launch"], 3),
                                             "padding_frac": round(float((gs.scores == -float("inf")).mean()), 3)}
        log(f"[short_context] cold {cold['us_per_launch']:.3f} us, warm {hot['us_per_launch']:.3f} us")
    if "prefill" in configs:
        extra["prefill"] = bench_prefill(run, args.trials)
        log(f"[prefill] {extra['prefill']}")
    if "fused" in configs:
        extra["fused_merge"] = bench_fused(run, args.steps, args.warmup, args.trials)
        log(f"[fused] {extra['fused_merge']}")
    if "local" in configs:
        extra["local_topk"] = bench_local(run, args.steps, args.warmup, args.trials)
        log(f"[local] {extra['local_topk']}")

    if cpu_extra is not None:
        extra["cpu_oracle"] = cpu_extra
        gpu_us = {"large": us}
        if "decode_latency_us" in extra:
            gpu_us["decode_rows16"] = extra["decode_latency_us"]["rows16"]["cold_us"]
        if "tie_heavy_latency_us" in extra:
            gpu_us["tie_heavy"] = extra["tie_heavy_latency_us"]["cold_us"]
        extra["cpu_oracle"]["gpu_us_same_batches"] = gpu_us

    traffic = traffic_record(us)
    line = {
        "metric": METRIC,
        "value": g.rows * g.num_cand / (us * 1e-6),
        "unit": "candidates/s",
        "n_gpus": 1,
        "steps": res["launches"] * args.trials,
        "warmup": args.warmup,
        "ms_per_step": us * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": "large: 256 rows x 8192 candidates (DCP 4 x local K 2048), K 2048, scores U(-10,10), "
                               "inputs rotated through a 576+ MiB pool (HBM-cold)",
                   "rows": g.rows, "num_cand": g.num_cand, "k": g.k},
        "us_per_launch": us,
        "timing": {"launches_per_trial": res["launches"], "trials": args.trials, "steps_requested": args.steps,
                   "stat": "median over trials of the per-launch time of one graph replay"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": "stable_topk_kernel<512, 2, 16, full, GatheredSource, PairSink>", "algorithmic_bytes_per_launch": per_launch_bytes},
        "cpu_baseline": cpu,
        "context": {"pages_selector_us_rows256_c8192": 15.459,
                    "pages_note": "PR #47348 Benchmarks, median of 7x200 launches; hardware and K not stated"},
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
