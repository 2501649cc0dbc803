"""CSA2 (Compressed Sparse Attention 2) hot path for AMD MI355X (gfx950).

The compute lives in libcsa2.so (C ABI in include/csa2.h); `csa2` is its Python binding.
"""
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2.so")


def load():
    """Import the binding (raises if libcsa2.so has not been built)."""
    from . import csa2
    return csa2
