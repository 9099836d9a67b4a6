"""Fast-multipole Newtonian gravity on one AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libmbg_fmm.so`` built from ``csrc/``
(hand-written HIP kernels); ``Plan`` in ``fmm.py`` is its thin Python binding.
``workloads`` generates seeded synthetic particle sets.  The binding is loaded
lazily so that input generation works without the GPU library.
"""
from __future__ import annotations

__all__ = ["Plan", "FmmError", "direct", "workloads"]


def __getattr__(name):
    if name in ("Plan", "FmmError", "direct"):
        from . import fmm
        return getattr(fmm, name)
    raise AttributeError(name)
