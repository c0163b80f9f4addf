"""Dual-Flow Transformer grouped decode step on MI355X (gfx950).

The product is the C-ABI library ``libdualflow.so`` (include/dualflow.h);
``_abi`` is its ctypes binding and ``runtime`` places a workload's tensors on
the GPU and calls it. There is no CPU fallback: a missing library raises.
"""
from . import _abi  # noqa: F401
from ._abi import lib  # noqa: F401

__all__ = ["_abi", "lib"]
