"""W4A8 mixture-of-experts routed-expert layer for MI355X (gfx950).

The layer is a C-ABI library of HIP kernels (``libw4a8moe.so``, declared in
``include/w4a8_moe.h``); ``ops`` is its thin Python binding and ``layer``
chains the calls.  Importing this package loads nothing native: the library
is loaded on first use by ``ops`` and its absence is an error there.
"""
__all__ = ["ops", "layer", "workloads"]
