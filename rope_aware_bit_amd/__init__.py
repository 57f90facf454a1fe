"""rope_aware_bit_amd — packed low-bit KV cache with RoPE-aware bit allocation on MI355X.

The product is the C-ABI library libkvq.so (include/kvq.h), built from the HIP
sources in csrc/ for gfx950.  ``rope_aware_bit_amd.kvq`` is a thin ctypes
binding over it; importing it fails loudly when the library is not built.
"""
__all__ = ["kvq", "build"]
