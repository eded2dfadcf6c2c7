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

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, ESCRATCH = 0, -1, -2, -3, -4, -5
MERGE_ROWS = 1024
MAX_CANDIDATES = 16384
MAX_ROWS = 4194303
FUSED_MAX_RANKS = 16
WORKSPACE_ALIGN = 256
STATIC_SCRATCH_BYTES = 64 << 20
SPLIT_MAX_PARTS = 8

_lib = None


class DcpTopkError(RuntimeError):
    def __init__(self, func: str, status: int):
        super().__init__(f"{func} failed: {status_string(status)} (status {status})")
        self.status = status


def _p(x):
    return ctypes.c_void_p(x)


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdcptopk.so and declare its signatures (raises if it is missing).
    Every wrapper below calls through the library loaded here."""
    global _lib
    if _lib is None:
        _lib = open_library(path)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """Open a build of the library at `path` with its signatures declared,
    without making it the one the wrappers use."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m stable_top_selection_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.dcp_topk_pack.argtypes = [vp, vp, i64, vp, i32, i32, i32, vp, i64, vp]
    lib.dcp_topk_pack.restype = ctypes.c_int
    lib.dcp_topk_select.argtypes = [vp, i32, i32, i32, vp, vp]
    lib.dcp_topk_select.restype = ctypes.c_int
    lib.dcp_topk_select_split_workspace_bytes.argtypes = [i32, i32, i32]
    lib.dcp_topk_select_split_workspace_bytes.restype = sz
    lib.dcp_topk_select_split.argtypes = [vp, i32, i32, i32, i32, vp, sz, vp, vp]
    lib.dcp_topk_select_split.restype = ctypes.c_int
    lib.dcp_topk_merge_workspace_bytes.argtypes = [i32, i32, i32]
    lib.dcp_topk_merge_workspace_bytes.restype = sz
    lib.dcp_topk_merge_chunked.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, sz, vp, vp]
    lib.dcp_topk_merge_chunked.restype = ctypes.c_int
    lib.dcp_topk_merge_chunked_static.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp]
    lib.dcp_topk_merge_chunked_static.restype = ctypes.c_int
    lib.dcp_topk_merge_fused.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp]
    lib.dcp_topk_merge_fused.restype = ctypes.c_int
    lib.dcp_topk_local.argtypes = [vp, i64, vp, i32, i32, i32, vp, vp, i64, vp]
    lib.dcp_topk_local.restype = ctypes.c_int
    lib.dcp_topk_status_string.argtypes = [ctypes.c_int]
    lib.dcp_topk_status_string.restype = ctypes.c_char_p
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


def _require_rows(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    """A 2-D device tensor whose rows are contiguous (any row stride >= width)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype or t.dim() != 2:
        raise ValueError(f"{name} must be {dtype} with 2 dims, got {t.dtype} {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous rows")


def _row_stride(t: torch.Tensor) -> int:
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)


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


def select_split_workspace_bytes(rows: int, num_cand: int, parts: int) -> int:
    return int(load_library().dcp_topk_select_split_workspace_bytes(rows, num_cand, parts))


def select_split_workspace(rows: int, num_cand: int, parts: int, device) -> torch.Tensor:
    """A zero-filled workspace for ``select_split`` (reusable by later calls on
    the same stream: every call leaves its counters at zero)."""
    return torch.zeros(max(select_split_workspace_bytes(rows, num_cand, parts), 1), dtype=torch.uint8, device=device)


def select_split(cand: torch.Tensor, k: int, parts: int, workspace: torch.Tensor | None = None,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """``select`` with each row spread over ``parts`` workgroups (for few rows)."""
    lib = load_library()
    _require(cand, "cand", torch.int32, 3)
    rows, c, two = cand.shape
    if two != 2:
        raise ValueError("cand must be (rows, C, 2)")
    if workspace is None:
        workspace = select_split_workspace(rows, c, parts, cand.device)
    _require(workspace, "workspace", torch.uint8, 1)
    if out is None:
        out = torch.empty((rows, max(int(k), 0), 2), dtype=torch.int32, device=cand.device)
    _require(out, "out", torch.int32, 3)
    if tuple(out.shape) != (rows, k, 2):
        raise ValueError(f"out must be ({rows}, {k}, 2)")
    _check("dcp_topk_select_split",
           lib.dcp_topk_select_split(_p(cand.data_ptr()), rows, c, int(k), int(parts), _p(workspace.data_ptr()),
                                     workspace.numel(), _p(out.data_ptr()), _stream(cand.device)))
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
    rows, local_k = _check_ranks(local_scores, local_idx, row_starts)
    device = local_scores[0].device
    need = merge_workspace_bytes(rows, dcp, local_k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _require(workspace, "workspace", torch.uint8, 1)
    if out is None:
        out = torch.empty((rows, k, 2), dtype=torch.int32, device=device)
    _require(out, "out", torch.int32, 3)
    arrays = _RankArrays(local_scores, local_idx, row_starts, rank_offsets)  # alive for the call
    sp, ip, rp, offs = arrays.args()
    _check("dcp_topk_merge_chunked",
           lib.dcp_topk_merge_chunked(sp, ip, rp, offs, dcp, rows, local_k, int(k), _p(workspace.data_ptr()),
                                      workspace.numel(), _p(out.data_ptr()), _stream(device)))
    return out


def merge_chunked_static(local_scores: Sequence[torch.Tensor], local_idx: Sequence[torch.Tensor],
                         row_starts: Sequence[torch.Tensor], rank_offsets: Sequence[int], k: int,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """The chunked merge with the library's static per-GPU workspace (no
    allocation in the library): same result as merge_chunked.  Calls that
    overlap in time on one GPU race."""
    lib = load_library()
    dcp = len(local_scores)
    rows, local_k = _check_ranks(local_scores, local_idx, row_starts)
    device = local_scores[0].device
    if out is None:
        out = torch.empty((rows, k, 2), dtype=torch.int32, device=device)
    _require(out, "out", torch.int32, 3)
    arrays = _RankArrays(local_scores, local_idx, row_starts, rank_offsets)  # alive for the call
    sp, ip, rp, offs = arrays.args()
    _check("dcp_topk_merge_chunked_static",
           lib.dcp_topk_merge_chunked_static(sp, ip, rp, offs, dcp, rows, local_k, int(k), _p(out.data_ptr()),
                                             _stream(device)))
    return out


def _check_ranks(local_scores, local_idx, row_starts) -> tuple[int, int]:
    dcp = len(local_scores)
    if not (len(local_idx) == len(row_starts) == dcp) or dcp < 1:
        raise ValueError("one scores / idx / row_starts / offset per rank")
    rows, local_k = local_scores[0].shape
    for r in range(dcp):
        _require(local_scores[r], f"local_scores[{r}]", torch.float32, 2)
        _require(local_idx[r], f"local_idx[{r}]", torch.int32, 2)
        _require(row_starts[r], f"row_starts[{r}]", torch.int32, 1)
        if tuple(local_scores[r].shape) != (rows, local_k) or tuple(local_idx[r].shape) != (rows, local_k) \
                or row_starts[r].shape[0] != rows:
            raise ValueError("inconsistent shapes")
    return rows, local_k


class _RankArrays:
    """Host arrays of the ranks' device pointers, kept alive for one call."""

    def __init__(self, local_scores, local_idx, row_starts, rank_offsets):
        dcp = len(local_scores)
        if len(rank_offsets) != dcp:
            raise ValueError("one rank offset per rank")
        ptrs = ctypes.c_void_p * dcp
        self.sp = ptrs(*[t.data_ptr() for t in local_scores])
        self.ip = ptrs(*[t.data_ptr() for t in local_idx])
        self.rp = ptrs(*[t.data_ptr() for t in row_starts])
        self.offs = (ctypes.c_int32 * dcp)(*[int(x) for x in rank_offsets])

    def args(self):
        return [ctypes.cast(a, ctypes.c_void_p) for a in (self.sp, self.ip, self.rp, self.offs)]


def merge_fused(local_scores: Sequence[torch.Tensor], local_idx: Sequence[torch.Tensor],
                row_starts: Sequence[torch.Tensor], rank_offsets: Sequence[int], k: int,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """The merge without a gathered buffer: select straight from every rank's
    local arrays (local_k a multiple of 64).  Same result as merge_chunked."""
    lib = load_library()
    rows, local_k = _check_ranks(local_scores, local_idx, row_starts)
    device = local_scores[0].device
    if out is None:
        out = torch.empty((rows, k, 2), dtype=torch.int32, device=device)
    _require(out, "out", torch.int32, 3)
    if tuple(out.shape) != (rows, k, 2):
        raise ValueError(f"out must be ({rows}, {k}, 2)")
    arrays = _RankArrays(local_scores, local_idx, row_starts, rank_offsets)  # alive for the call
    sp, ip, rp, offs = arrays.args()
    _check("dcp_topk_merge_fused",
           lib.dcp_topk_merge_fused(sp, ip, rp, offs, len(local_scores), rows, local_k, int(k),
                                    _p(out.data_ptr()), _stream(device)))
    return out


def local_topk(scores: torch.Tensor, k: int, lengths: torch.Tensor | None = None,
               out_scores: torch.Tensor | None = None, out_idx: torch.Tensor | None = None):
    """Per row of ``scores`` (rows, num_cols) fp32 (rows contiguous, any row
    stride): the k best of the first lengths[row] columns (all without
    ``lengths``), ties to the lowest column, in column order, then (-inf, -1).
    Returns (out_scores (rows, k) fp32, out_idx (rows, k) int32)."""
    lib = load_library()
    _require_rows(scores, "scores", torch.float32)
    rows, num_cols = scores.shape
    device = scores.device
    if lengths is not None:
        _require(lengths, "lengths", torch.int32, 1)
        if lengths.shape[0] != rows:
            raise ValueError("lengths must have one entry per row")
    if out_scores is None:
        out_scores = torch.empty((rows, k), dtype=torch.float32, device=device)
    if out_idx is None:
        out_idx = torch.empty((rows, k), dtype=torch.int32, device=device)
    _require_rows(out_scores, "out_scores", torch.float32)
    _require_rows(out_idx, "out_idx", torch.int32)
    if tuple(out_scores.shape) != (rows, k) or tuple(out_idx.shape) != (rows, k):
        raise ValueError(f"outputs must be ({rows}, {k})")
    out_stride = _row_stride(out_scores)
    if _row_stride(out_idx) != out_stride:
        raise ValueError("out_scores and out_idx must share a row stride")
    _check("dcp_topk_local",
           lib.dcp_topk_local(_p(scores.data_ptr()), _row_stride(scores),
                              _p(lengths.data_ptr() if lengths is not None else 0), rows, num_cols, int(k),
                              _p(out_scores.data_ptr()), _p(out_idx.data_ptr()), out_stride, _stream(device)))
    return out_scores, out_idx


def split(cand: torch.Tensor):
    """(rows, C, 2) int32 candidates -> (scores fp32, ids int32) views."""
    return cand[..., 0].contiguous().view(torch.float32), cand[..., 1].contiguous()
