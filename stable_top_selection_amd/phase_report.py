"""Phase timeline of the select kernel on one MI355X, from the phase-stamp
build of the library (``libdcptopk_phases.so``, compiled by ``build_all``).

In that build lane 0 of the first and of the last wave of every workgroup
reads the shader clock (``s_memtime``) at each phase boundary of the select
kernel.  This script runs ``dcp_topk_select`` on a workload, reads the stamps
of every workgroup (one row each) and prints, per phase, the median over the
rows of the time from the start of wave 0 to the phase's end in the last wave
(the later of the two) and the median length of the phase, in shader-clock
cycles.  ``cold`` samples read inputs that no launch has touched since a pass
over more than twice the Infinity Cache plus L2; ``warm`` samples repeat the
previous launch's input.

    python -m stable_top_selection_amd.phase_report [--workload large|decode16|tie_heavy|fused] [--samples 8]

``fused`` runs the fused merge (dcp_topk_merge_fused) on the large shape
(256 rows, DCP 4 x local K 2048), whose kernel reads every rank's local
arrays in place; the others run dcp_topk_select on a gathered buffer.

The stamps cost a few instructions per boundary, so the absolute times are
slightly above the product build's; the product's timing is bench.py's.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PHASES = ["kernel arguments read, row addresses computed", "loads issued, LDS cleared, first barrier",
          "pass-0 atomics issued", "pass-0 barrier", "digit search", "list built", "first list pass",
          "threshold resolved", "selection flags", "ranks", "staging writes", "count exchange", "stores issued"]
SLOTS = 16  # stamps per wave in the library's array
STAMP_ROWS = 1024
POOL_BYTES = 2 * (256 + 32) * (1 << 20)


def _timelines(st: np.ndarray, rows: int):
    """Per row: (end of each phase, the later of the two stamped waves, from
    wave 0's start; the last wave's lag behind the first at that boundary);
    phases the row did not pass are None."""
    st = st.reshape(STAMP_ROWS, 2, SLOTS)[:rows].astype(np.int64)
    out = []
    for r in range(rows):
        t0 = st[r, 0, 0]
        ends = []
        for p in range(1, len(PHASES) + 1):
            a, b = st[r, 0, p], st[r, 1, p]
            ends.append(None if (a == 0 and b == 0) else (int(max(a, b) - t0), int(b - a)))
        out.append(ends)
    return out


def _start_lags(st: np.ndarray, rows: int):
    """Per row: how many cycles after wave 0 the last wave started."""
    st = st.reshape(STAMP_ROWS, 2, SLOTS)[:rows].astype(np.int64)
    return [int(st[r, 1, 0] - st[r, 0, 0]) for r in range(rows)]


def _summarise(lines):
    """Per phase: rows that passed it, and over them the median end, median
    length (from the previous phase the row passed) and median lag of the
    last wave behind the first."""
    res = []
    for p in range(len(PHASES)):
        ends = [ln[p][0] for ln in lines if ln[p] is not None]
        lags = [ln[p][1] for ln in lines if ln[p] is not None]
        lens = []
        for ln in lines:
            if ln[p] is None:
                continue
            prev = next((ln[q][0] for q in range(p - 1, -1, -1) if ln[q] is not None), 0)
            lens.append(ln[p][0] - prev)
        med = lambda x: statistics.median(x) if x else None  # noqa: E731
        res.append((len(ends), med(ends), med(lens), med(lags)))
    return res


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", default="large", choices=["large", "decode16", "tie_heavy", "fused"])
    ap.add_argument("--samples", type=int, default=8, help="launches stamped per mode")
    ap.add_argument("--lib", default=None, help="a phase-stamp build of the library (default: the package's)")
    args = ap.parse_args()

    import torch

    from stable_top_selection_amd import binding as B
    from stable_top_selection_amd import build as BLD
    from stable_top_selection_amd import workloads as W

    lib = B.open_library(args.lib or BLD.PHASES_LIB_PATH)
    lib.dcptopk_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.dcptopk_phase_stamps.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    if args.workload == "fused":
        sh = W.fused()
        rows, k, name, num_cand = sh.rows, sh.k, sh.name, sh.dcp * sh.local_k
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
        per = sh.dcp * sh.rows * sh.local_k * 8
        n = max(args.samples + 1, -(-POOL_BYTES // per))
        # a pool of copies of the ranks' arrays: each entry holds the device
        # tensors (kept alive here) and the host arrays of their pointers
        pool = []
        for _ in range(n):
            arrays = ([to(sh.scores[r]) for r in range(sh.dcp)], [to(sh.local_idx[r]) for r in range(sh.dcp)],
                      [to(sh.row_starts[r]) for r in range(sh.dcp)])
            pool.append((arrays, B._RankArrays(*arrays, [int(x) for x in sh.rank_offsets])))
        out = torch.empty((rows, k, 2), dtype=torch.int32, device=dev)

        def launch(entry):
            st = lib.dcp_topk_merge_fused(*entry[1].args(), sh.dcp, rows, sh.local_k, k,
                                          ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream))
            if st != 0:
                raise RuntimeError(f"dcp_topk_merge_fused: {B.status_string(st)}")
    else:
        g = {"large": W.large, "decode16": lambda: W.decode(16), "tie_heavy": W.tie_heavy}[args.workload]()
        rows, k, name, num_cand = g.rows, g.k, g.name, g.num_cand
        inter = torch.from_numpy(g.interleaved()).to(dev)
        per = inter.numel() * 4
        n = max(args.samples + 1, -(-POOL_BYTES // per))
        pool = [inter.clone() for _ in range(n)]
        out = torch.empty((rows, k, 2), dtype=torch.int32, device=dev)

        def launch(buf):
            st = lib.dcp_topk_select(ctypes.c_void_p(buf.data_ptr()), rows, num_cand, k,
                                     ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream))
            if st != 0:
                raise RuntimeError(f"dcp_topk_select: {B.status_string(st)}")
    if rows > STAMP_ROWS:
        raise SystemExit(f"at most {STAMP_ROWS} rows are stamped")
    stamps = np.zeros(STAMP_ROWS * 2 * SLOTS, dtype=np.uint64)

    def read():
        e = lib.dcptopk_phase_stamps(ctypes.c_void_p(stamps.ctypes.data), stamps.nbytes)
        if e != 0:
            raise RuntimeError(f"dcptopk_phase_stamps: {e}")
        return _timelines(stamps, rows)

    # the pool's buffers were written in order, so the earliest ones have left
    # the caches by the time the last is written: cold samples take those
    torch.cuda.synchronize()
    read()  # clear
    cold, warm, lag_cold, lag_warm = [], [], [], []
    for s in range(args.samples):
        launch(pool[s])
        cold += read()
        lag_cold += _start_lags(stamps, rows)
        launch(pool[s])
        warm += read()
        lag_warm += _start_lags(stamps, rows)
    print(f"workload {name}: {rows} rows x {num_cand} candidates, k {k}; "
          f"{args.samples} launches per mode, medians over rows x launches, shader-clock cycles from wave 0's start")
    print()
    print("| Phase (end, later of the first and last wave) | Rows x launches passing | Cold: end | Cold: length | "
          "Cold: last wave behind first | Warm: end | Warm: length |")
    print("|---|---|---|---|---|---|---|")
    for name, c, w in zip(PHASES, _summarise(cold), _summarise(warm)):
        fmt = lambda x: "-" if x is None else f"{x:,.0f}"  # noqa: E731
        print(f"| {name} | {c[0]} / {len(cold)} | {fmt(c[1])} | {fmt(c[2])} | {fmt(c[3])} | {fmt(w[1])} | "
              f"{fmt(w[2])} |")
    print()
    print(f"Start of the workgroup's last wave behind its wave 0 (median, cycles): cold "
          f"{statistics.median(lag_cold):,.0f}, warm {statistics.median(lag_warm):,.0f}")


if __name__ == "__main__":
    main()
