"""NOSA per-decode-step block-sparse attention path for AMD MI355X (gfx950).

The compute path is libnosa.so (hand-written HIP kernels behind the C ABI in
include/nosa.h); ``_lib`` binds it with ctypes and ``pipeline`` sequences the
calls of one decode step. Importing this package fails if libnosa.so has not
been built: there is no fallback implementation.
"""
from . import _lib  # noqa: F401  (loads libnosa.so or raises ImportError)
from ._lib import NosaError  # noqa: F401
from .hostmem import PinnedBuffer  # noqa: F401
from .pipeline import DecodeLayer, block_offsets, pack_blocks, unpack_blocks  # noqa: F401

__all__ = ["DecodeLayer", "NosaError", "PinnedBuffer", "block_offsets", "pack_blocks",
           "unpack_blocks"]
