"""Focus attention forward path for AMD Instinct MI355X (gfx950).

Focus ("Why Attend to Everything? Focus is the Key", arXiv 2604.03260) keeps,
for each query, exact softmax over a local window of recent keys plus the
older keys that share one of its top-k centroid groups.  This package holds
the hand-written HIP kernels behind a C ABI (``libfocus.so``, declared in
``include/focus.h``) and a thin ctypes binding with the same call names.

Importing the package loads nothing; the first call into the binding loads
``libfocus.so`` and raises if it has not been built.
"""
from .workloads import WORKLOADS, Workload  # noqa: F401

__all__ = ["WORKLOADS", "Workload"]
