"""MI355X-native stable top-K selection for the DCP sparse-indexer merge.

The compute path lives in ``libdcptopk.so`` (hand-written HIP for gfx950,
C ABI declared in ``include/libdcptopk.h``).  ``stable_top_selection_amd.binding``
is a thin ctypes layer over it that takes torch device tensors; importing this
package does not load the library.
"""

__all__ = ["binding", "workloads"]
