"""MI355X-native block-causal 3D-RoPE joint attention with a prefix KV cache.

The library is libqi.so (C ABI in include/qi.h, HIP kernels for gfx950); ``qi`` is its
ctypes binding and ``runtime`` a thin torch helper for device buffers and streams.
"""
from . import qi  # noqa: F401

__all__ = ["qi"]
