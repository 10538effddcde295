"""BeaconKV eviction hot path on AMD MI355X (gfx950).

The compute lives in ``libbkv.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/bkv.h``).  ``lib()`` returns the ctypes binding, which
only marshals torch tensors into pointers and raises if the library is
missing; there is no CPU fallback.
"""
from . import configs  # noqa: F401

__all__ = ["lib", "configs"]


def lib():
    from . import bkv

    return bkv.load()
