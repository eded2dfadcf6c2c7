"""Thin ctypes binding of libdcptopk (the C ABI in ``include/libdcptopk.h``).

Argument marshalling only: every step of the path runs in the HIP library.
torch provides device memory and the current HIP stream.  Candidate tensors
are int32 of shape (rows, C, 2): [..., 0] holds the fp32 score bits and
[..., 1] the global token id, which is the library's 8-byte candidate layout.

The library must be built (``python -m stable_top_selection_amd.build``);
there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Sequence

import torch

from .build import INCLUDE, LIB_PATH

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
MERGE_ROWS = 1024
MAX_CANDIDATES = 16384
WORKSPACE_ALIGN = 256

_lib = None


class DcpTopkError(RuntimeError):
    def __init__(self, func: str, status: int):
        super().__init__(f"{func} failed: {status_string(status)} (status {status})")
        self.status = status


def _p(x):
    return ctypes.c_void_p(x)


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdcptopk.so and declare its signatures (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m stable_top_selection_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.dcp_topk_pack.argtypes = [vp, vp, i64, vp, i32, i32, i32, vp, i64, vp]
    lib.dcp_topk_pack.restype = ctypes.c_int
    lib.dcp_topk_select.argtypes = [vp, i32, i32, i32, vp, vp]
    lib.dcp_topk_select.restype = ctypes.c_int
    lib.dcp_topk_merge_workspace_bytes.argtypes = [i32, i32, i32]
    lib.dcp_topk_merge_workspace_bytes.restype = sz
    lib.dcp_topk_merge_chunked.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, sz, vp, vp]
    lib.dcp_topk_merge_chunked.restype = ctypes.c_int
    lib.dcp_topk_status_string.argtypes = [ctypes.c_int]
    lib.dcp_topk_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions ``include/libdcptopk.h`` declares."""
    with open(os.path.join(INCLUDE, "libdcptopk.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dcp_topk_[a-z_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return load_library().dcp_topk_status_string(int(status)).decode()


def _check(func: str, status: int) -> None:
    if status != OK:
        raise DcpTopkError(func, status)


def _stream(device: torch.device) -> ctypes.c_void_p:
    return _p(torch.cuda.current_stream(device).cuda_stream)


def _require(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype or t.dim() != ndim:
        raise ValueError(f"{name} must be {dtype} with {ndim} dims, got {t.dtype} {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def candidates_from(scores: torch.Tensor, ids: torch.Tensor) -> torch.Tensor:
    """(rows, C) fp32 scores + (rows, C) int32 ids -> (rows, C, 2) int32 candidates."""
    return torch.stack([scores.contiguous().view(torch.int32), ids.to(torch.int32)], dim=-1).contiguous()


def select(cand: torch.Tensor, k: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Stable top-k of every row of ``cand`` (rows, C, 2) int32 -> (rows, k, 2) int32."""
    lib = load_library()
    _require(cand, "cand", torch.int32, 3)
    rows, c, two = cand.shape
    if two != 2:
        raise ValueError("cand must be (rows, C, 2)")
    if out is None:
        out = torch.empty((rows, max(int(k), 0), 2), dtype=torch.int32, device=cand.device)
    _require(out, "out", torch.int32, 3)
    if tuple(out.shape) != (rows, k, 2):
        raise ValueError(f"out must be ({rows}, {k}, 2)")
    _check("dcp_topk_select",
           lib.dcp_topk_select(_p(cand.data_ptr()), rows, c, int(k), _p(out.data_ptr()), _stream(cand.device)))
    return out


def pack(local_scores: torch.Tensor, local_idx: torch.Tensor, row_starts: torch.Tensor, rank_offset: int,
         dst: torch.Tensor, column: int = 0) -> torch.Tensor:
    """Pack one rank's (T, local_k) scores/indices into ``dst`` (T, C, 2) int32
    at columns [column, column + local_k).  Returns ``dst``."""
    lib = load_library()
    _require(local_scores, "local_scores", torch.float32, 2)
    _require(local_idx, "local_idx", torch.int32, 2)
    _require(row_starts, "row_starts", torch.int32, 1)
    _require(dst, "dst", torch.int32, 3)
    rows, local_k = local_scores.shape
    if tuple(local_idx.shape) != (rows, local_k) or row_starts.shape[0] != rows or dst.shape[0] != rows:
        raise ValueError("inconsistent shapes")
    if not (0 <= column and column + local_k <= dst.shape[1]):
        raise ValueError("column range outside dst")
    dst_ptr = dst.data_ptr() + 8 * column
    _check("dcp_topk_pack",
           lib.dcp_topk_pack(_p(local_scores.data_ptr()), _p(local_idx.data_ptr()), local_k,
                             _p(row_starts.data_ptr()), int(rank_offset), rows, local_k, _p(dst_ptr),
                             dst.shape[1], _stream(dst.device)))
    return dst


def merge_workspace_bytes(rows: int, dcp: int, local_k: int) -> int:
    return int(load_library().dcp_topk_merge_workspace_bytes(rows, dcp, local_k))


def merge_chunked(local_scores: Sequence[torch.Tensor], local_idx: Sequence[torch.Tensor],
                  row_starts: Sequence[torch.Tensor], rank_offsets: Sequence[int], k: int,
                  workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """The whole one-GPU merge: pack every rank and select, 1024 rows at a time."""
    lib = load_library()
    dcp = len(local_scores)
    if not (len(local_idx) == len(row_starts) == len(rank_offsets) == dcp) or dcp < 1:
        raise ValueError("one scores / idx / row_starts / offset per rank")
    rows, local_k = local_scores[0].shape
    for r in range(dcp):
        _require(local_scores[r], f"local_scores[{r}]", torch.float32, 2)
        _require(local_idx[r], f"local_idx[{r}]", torch.int32, 2)
        _require(row_starts[r], f"row_starts[{r}]", torch.int32, 1)
        if tuple(local_scores[r].shape) != (rows, local_k) or tuple(local_idx[r].shape) != (rows, local_k) \
                or row_starts[r].shape[0] != rows:
            raise ValueError("inconsistent shapes")
    device = local_scores[0].device
    need = merge_workspace_bytes(rows, dcp, local_k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _require(workspace, "workspace", torch.uint8, 1)
    if out is None:
        out = torch.empty((rows, k, 2), dtype=torch.int32, device=device)
    _require(out, "out", torch.int32, 3)
    ptrs = ctypes.c_void_p * dcp
    sp = ptrs(*[t.data_ptr() for t in local_scores])
    ip = ptrs(*[t.data_ptr() for t in local_idx])
    rp = ptrs(*[t.data_ptr() for t in row_starts])
    offs = (ctypes.c_int32 * dcp)(*[int(x) for x in rank_offsets])
    _check("dcp_topk_merge_chunked",
           lib.dcp_topk_merge_chunked(ctypes.cast(sp, ctypes.c_void_p), ctypes.cast(ip, ctypes.c_void_p),
                                      ctypes.cast(rp, ctypes.c_void_p), ctypes.cast(offs, ctypes.c_void_p), dcp,
                                      rows, local_k, int(k), _p(workspace.data_ptr()), workspace.numel(),
                                      _p(out.data_ptr()), _stream(device)))
    return out


def split(cand: torch.Tensor):
    """(rows, C, 2) int32 candidates -> (scores fp32, ids int32) views."""
    return cand[..., 0].contiguous().view(torch.float32), cand[..., 1].contiguous()
