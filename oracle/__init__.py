"""CPU oracle for the DCP stable top-K merge.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path, which
runs entirely in the HIP library.  See ``oracle/stable_topk.py`` for the
definitions and the readings of the pages they follow.
"""
from .stable_topk import (  # noqa: F401
    CANDIDATE_BYTES,
    INT32_MAX,
    MERGE_ROWS,
    gather_output_bytes,
    gather_rows,
    merge,
    merge_workspace_bytes,
    pack,
    pages_scratch_bytes,
    score_key,
    select,
    sort_key64,
)
