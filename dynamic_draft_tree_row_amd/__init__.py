"""Dynamic draft-tree round (EAGLE-2 expansion/rerank, CAST, Graft) for MI355X.

The round runs in the HIP kernels of libddt.so behind the C ABI of
include/ddt.h; this package is its thin Python binding plus a round driver.
Importing the package does not load the library; the first call does, and it
raises if libddt.so has not been built.
"""
from . import _lib  # noqa: F401

__all__ = ["api", "round_driver"]
