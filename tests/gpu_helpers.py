"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
(binding) and the CPU oracle on the same seeded inputs, compare bit for bit."""
from __future__ import annotations

import numpy as np
import torch

from oracle import stable_topk as O
from stable_top_selection_amd import binding as B

DEV = "cuda:0"


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_select(scores: np.ndarray, ids: np.ndarray, k: int, guard: int = 0, misalign: bool = False,
               split_parts: int = 0, workspace: torch.Tensor | None = None):
    """Select on the GPU; returns (score bits uint32, ids int32), each (rows, k).

    ``guard`` rows of canary candidates are placed before and after the output
    and must survive untouched; ``misalign`` starts the candidate buffer 8
    bytes past a 16-byte boundary (the 8-byte load path).  ``split_parts`` > 0
    selects through the split-row entry point with that many workgroups per
    row (in ``workspace`` if given, else a fresh zeroed one)."""
    rows, c = scores.shape
    inter = np.empty((rows, c, 2), np.int32)
    inter[..., 0] = scores.view(np.int32)
    inter[..., 1] = ids
    if misalign:
        flat = torch.zeros(rows * c * 2 + 2, dtype=torch.int32, device=DEV)
        flat[2:] = to_dev(inter.reshape(-1))
        cand = flat[2:].view(rows, c, 2)
        assert cand.data_ptr() % 16 == 8
    else:
        cand = to_dev(inter)
    canary = torch.tensor([0x5EED5EED, 0x0BADF00D], dtype=torch.int32, device=DEV)
    big = canary.repeat((rows + 2 * guard) * k).view(rows + 2 * guard, k, 2) if k > 0 else None
    out = big[guard:guard + rows]
    if split_parts:
        B.select_split(cand, k, split_parts, workspace=workspace, out=out)
    else:
        B.select(cand, k, out=out)
    torch.cuda.synchronize()
    if guard:
        g = big.cpu().numpy()
        assert np.all(g[:guard, :, 0] == 0x5EED5EED) and np.all(g[:guard, :, 1] == 0x0BADF00D), "wrote before out"
        assert np.all(g[guard + rows:, :, 0] == 0x5EED5EED) and np.all(g[guard + rows:, :, 1] == 0x0BADF00D), \
            "wrote after out"
    o = out.cpu().numpy()
    return o[..., 0].view(np.uint32).copy(), o[..., 1].copy()


def assert_select_parity(scores: np.ndarray, ids: np.ndarray, k: int, label: str = "", **kw) -> None:
    gb, gi = gpu_select(scores, ids, k, **kw)
    os_, oi = O.select(scores, ids, k)
    ob = os_.view(np.uint32)
    if not (np.array_equal(gb, ob) and np.array_equal(gi, oi)):
        bad = np.nonzero(~((gb == ob).all(1) & (gi == oi).all(1)))[0]
        r = int(bad[0])
        col = int(np.nonzero((gb[r] != ob[r]) | (gi[r] != oi[r]))[0][0])
        raise AssertionError(f"{label}: {len(bad)} rows differ; first row {r} col {col}: "
                             f"gpu ({gb[r, col]:#x}, {gi[r, col]}) oracle ({ob[r, col]:#x}, {oi[r, col]})")
