"""Replicated FP8 KV cache-store and device-epoch fence for MI355X (gfx950).

The product is ``libkvpub.so`` (C ABI in ``include/kvpub.h``; HIP sources in
``csrc/``).  ``kvpub`` is its thin ctypes binding, ``workloads`` the seeded
synthetic inputs used by the tests and the benchmark, ``build`` the in-tree
hipcc build.
"""
from . import kvpub  # noqa: F401

__all__ = ["kvpub"]
