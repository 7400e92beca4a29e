"""Block-sparse flash attention forward for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libbsattn.so`` built from ``csrc/``
(hand-written HIP kernels + host planner); ``bsattn`` is a thin ctypes
binding over it.  Importing this package does not load the library; the
first call that needs it does, and raises if it is missing.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads"]
