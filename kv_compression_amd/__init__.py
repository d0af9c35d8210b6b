"""MI355X-native store-h looped-decoder step (libtl.so, gfx950) and its Python binding.

The compute path is the HIP library behind include/tl.h; ``tl`` is the ctypes
binding (marshalling only). Importing this package does not touch the GPU.
"""
from . import tl  # noqa: F401

__all__ = ["tl"]
