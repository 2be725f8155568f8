"""Paged KV cache and paged decode attention for AMD MI355X (gfx950).

The work is done by ``libpkv.so`` (C ABI in ``include/pkv.h``: host block
allocator plus hand-written HIP kernels); ``pkv`` is its ctypes binding.
"""
from . import pkv  # noqa: F401
