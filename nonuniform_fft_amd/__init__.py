"""MI355X (gfx950) 1D/2D/3D type 1 / type 2 nonuniform FFT.

The transform runs in the HIP library libnufft_amd.so behind the C ABI of
include/nufft_amd.h; `Plan` is a thin ctypes binding over it that takes torch
device tensors and the current torch stream.
"""
from ._native import (METHOD_AUTO, METHOD_GM_SORT, METHOD_SM, NUFFT_ERR_ALLOC, NUFFT_ERR_BAD_ARG,  # noqa: F401
                      NUFFT_ERR_BAD_STATE, NUFFT_ERR_FFT, NUFFT_ERR_HIP, NUFFT_ERR_POINTS, NUFFT_ERR_UNSUPPORTED,
                      NUFFT_OK, NUFFT_WARN_EPS_CLAMPED, NufftError, Plan, load_library)

__all__ = ["Plan", "NufftError", "load_library", "METHOD_AUTO", "METHOD_GM_SORT", "METHOD_SM", "NUFFT_OK",
           "NUFFT_WARN_EPS_CLAMPED", "NUFFT_ERR_BAD_ARG", "NUFFT_ERR_BAD_STATE", "NUFFT_ERR_ALLOC", "NUFFT_ERR_HIP",
           "NUFFT_ERR_FFT", "NUFFT_ERR_POINTS", "NUFFT_ERR_UNSUPPORTED"]
