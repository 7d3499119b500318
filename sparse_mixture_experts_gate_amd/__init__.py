"""MI355X (gfx950) trainable sparse mixture-of-experts layer.

The layer runs in libmoe.so (HIP kernels behind a C ABI, include/moe.h).
This package holds the ctypes binding (`_lib`, same entry-point names as the
C ABI), the in-tree build script (`build`) and the seeded workload shapes and
inputs (`workloads`).  torch provides device memory and streams only.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads", "lib"]


def lib():
    """The ctypes binding; raises if libmoe.so has not been built."""
    from . import _lib
    _lib.load()
    return _lib
