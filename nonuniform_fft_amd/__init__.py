"""MI355X (gfx950) 1D/2D/3D type 1 / type 2 nonuniform FFT.

The transform runs in the HIP library libnufft_amd.so behind the C ABI of
include/nufft_amd.h; `Plan` is a thin ctypes binding over it that takes torch
device tensors and the current torch stream.
"""
from ._native import (METHOD_AUTO, METHOD_GM_SORT, METHOD_SM, NufftError, Plan,  # noqa: F401
                      load_library)

__all__ = ["Plan", "NufftError", "load_library", "METHOD_AUTO", "METHOD_GM_SORT", "METHOD_SM"]
