"""libbdattn: block-diffusion attention over a KV cache on MI355X (gfx950).

The product is the C-ABI shared library ``libbdattn.so`` (header
``include/bdattn.h``); ``bdattn`` is its ctypes binding.
"""
from . import bdattn  # noqa: F401

__all__ = ["bdattn"]
