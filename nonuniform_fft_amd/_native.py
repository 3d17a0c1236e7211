"""ctypes binding of the C ABI in include/nufft_amd.h (argument marshalling only).

Every step of the transform runs in the HIP library libnufft_amd.so; this module only
checks tensor shapes/dtypes/devices on the host and passes device pointers and the
current torch stream.  Importing it fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libnufft_amd.so")

# symbol -> (restype, argtypes); mirrors include/nufft_amd.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_D = ctypes.c_double


class NufftOpts(ctypes.Structure):
    _fields_ = [("method", ctypes.c_int), ("bin", ctypes.c_int * 3), ("subproblem_cap", ctypes.c_int),
                ("max_device_bytes", ctypes.c_size_t), ("timing", ctypes.c_int), ("max_batch", ctypes.c_int),
                ("upsampfac", ctypes.c_double)]


SIGNATURES = {
    "nufft_default_opts": (_I, [ctypes.POINTER(NufftOpts)]),
    "nufft_plan_create": (_I, [_I, _I, ctypes.POINTER(_L), _D, _I, _P, ctypes.POINTER(NufftOpts),
                               ctypes.POINTER(_P)]),
    "nufft_setpts": (_I, [_P, _L, _P, _P, _P]),
    "nufft_setpts_noalloc": (_I, [_P, _L, _P, _P, _P]),
    "nufft_setpts_type3": (_I, [_P, _L, _P, _P, _P, _L, _P, _P, _P]),
    "nufft_execute": (_I, [_P, _P, _P]),
    "nufft_execute_adjoint": (_I, [_P, _P, _P]),
    "nufft_execute_many": (_I, [_P, _I, _P, _P]),
    "nufft_execute_adjoint_many": (_I, [_P, _I, _P, _P]),
    "nufft_destroy": (_I, [_P]),
    "nufft_strerror": (ctypes.c_char_p, [_I]),
    "nufft_last_error": (ctypes.c_char_p, [_P]),
    "nufft_get_info": (_I, [_P, ctypes.POINTER(_L), ctypes.POINTER(_D)]),
    "nufft_get_stage_times": (_I, [_P, ctypes.POINTER(_D)]),
    "nufft_spread": (_I, [_P, _P, _P]),
    "nufft_interp": (_I, [_P, _P, _P]),
    "nufft_deconvolve": (_I, [_P, _P, _P]),
    "nufft_precorrect_pad": (_I, [_P, _P, _P]),
    "nufft_get_sort": (_I, [_P, _P, _P, _P]),
    "nufft_get_range_errors": (_I, [_P, ctypes.POINTER(_L)]),
}

NUFFT_OK = 0
NUFFT_WARN_EPS_CLAMPED = 1
NUFFT_ERR_BAD_ARG = -1
NUFFT_ERR_BAD_STATE = -2
NUFFT_ERR_ALLOC = -3
NUFFT_ERR_HIP = -4
NUFFT_ERR_FFT = -5
NUFFT_ERR_POINTS = -6
NUFFT_ERR_UNSUPPORTED = -7

METHOD_AUTO, METHOD_GM_SORT, METHOD_SM = 0, 1, 2

_lib = None


def load_library():
    """Load libnufft_amd.so (raise if it has not been built: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} not found: build the HIP library first "
                "(python -m nonuniform_fft_amd.build or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class NufftError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def _torch():
    import torch
    return torch


def _real_dtype(prec: int):
    torch = _torch()
    return torch.float32 if prec == 0 else torch.float64


def _complex_dtype(prec: int):
    torch = _torch()
    return torch.complex64 if prec == 0 else torch.complex128


class Plan:
    """A type 1, 2 or 3 NUFFT plan on the current HIP device (see include/nufft_amd.h).

    plan = Plan(1, (N1, N2, N3), eps=1e-5, precision="f32")
    plan.setpts(x, y, z)          # device tensors of M coordinates in [-pi, pi)
    plan.execute(c, f)            # type 1: c (M,) complex in, f (N3, N2, N1) complex out

    plan = Plan(3, d, eps)        # type 3 in d dimensions (N is the dimension count)
    plan.setpts_type3([x, y], [s, t])   # M sources, K targets (device tensors, any finite values)
    plan.execute(c, f)            # c (M,) in, f (K,) out
    """

    def __init__(self, nufft_type: int, N: Sequence[int], eps: float, precision: str = "f32",
                 stream=None, method: int = METHOD_AUTO, bins: Optional[Sequence[int]] = None,
                 subproblem_cap: int = 0, timing: bool = False, max_device_bytes: int = 0,
                 max_batch: int = 0, upsampfac: float = 0.0):
        lib = load_library()
        torch = _torch()
        if precision not in ("f32", "f64"):
            raise ValueError("precision must be 'f32' or 'f64'")
        self._lib = lib
        self._h = None
        self.type = int(nufft_type)
        if self.type == 3:
            d = int(N) if not hasattr(N, "__len__") else len(N)
            self.N = (1,) * d
        else:
            self.N = tuple(int(v) for v in N)
        self.dim = len(self.N)
        self.K = -1
        self.prec = 0 if precision == "f32" else 1
        opts = NufftOpts()
        lib.nufft_default_opts(ctypes.byref(opts))
        opts.method = int(method)
        if bins is not None:
            for i, b in enumerate(bins):
                opts.bin[i] = int(b)
        opts.subproblem_cap = int(subproblem_cap)
        opts.timing = 1 if timing else 0
        opts.max_device_bytes = int(max_device_bytes)
        opts.max_batch = int(max_batch)
        opts.upsampfac = float(upsampfac)
        if stream is None:
            stream = torch.cuda.current_stream()
        self._stream_obj = stream
        sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        Narr = (ctypes.c_int64 * max(self.dim, 1))(*self.N)
        h = ctypes.c_void_p()
        rc = lib.nufft_plan_create(self.type, self.dim, Narr, float(eps), self.prec, ctypes.c_void_p(sptr),
                                   ctypes.byref(opts), ctypes.byref(h))
        if rc < 0:
            raise NufftError(rc, lib.nufft_strerror(rc).decode())
        self.warning = rc
        self._h = h
        self.M = -1
        info = self.info()
        self.w = info["w"]
        self.n = info["n"]
        self.beta = info["beta"]

    # -- helpers -------------------------------------------------------------------------------
    def _check(self, rc: int):
        if rc < 0:
            detail = self._lib.nufft_last_error(self._h).decode()
            raise NufftError(rc, f"{self._lib.nufft_strerror(rc).decode()}: {detail}")
        return rc

    def _dev_tensor(self, t, dtype, shape, name):
        torch = _torch()
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
        if t.dtype != dtype:
            raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() != int(shape):
            raise ValueError(f"{name} must have {shape} elements, got {t.numel()}")
        return ctypes.c_void_p(t.data_ptr())

    @property
    def handle(self):
        return self._h

    @property
    def fine_cells(self) -> int:
        out = 1
        for v in self.n:
            out *= v
        return out

    @property
    def nmodes(self) -> int:
        out = 1
        for v in self.N:
            out *= v
        return out

    def info(self):
        ii = (ctypes.c_int64 * 20)()
        dd = (ctypes.c_double * 3)()
        self._check(self._lib.nufft_get_info(self._h, ii, dd))
        v = list(ii)
        return {"type": v[0], "dim": v[1], "precision": v[2], "w": v[3], "n": tuple(v[4:4 + self.dim]),
                "N": tuple(v[7:7 + self.dim]), "bins": tuple(v[10:10 + self.dim]), "nbins": v[13],
                "nsubproblems": v[14], "M": v[15], "cap": v[16], "method": v[17], "colw": v[18],
                "colstep": v[19],
                "beta": dd[0], "eps": dd[1], "sigma": dd[2]}

    # -- API -----------------------------------------------------------------------------------
    def setpts(self, x, y=None, z=None):
        coords = [x, y, z][:self.dim]
        if any(t is not None for t in [x, y, z][self.dim:]):
            raise ValueError(f"{self.dim}D plan takes {self.dim} coordinate array(s)")
        if any(t is None for t in coords):
            raise ValueError(f"{self.dim}D plan needs {self.dim} coordinate arrays")
        M = coords[0].numel()
        rd = _real_dtype(self.prec)
        ptrs = [self._dev_tensor(t, rd, M, name) for t, name in zip(coords, "xyz")]
        while len(ptrs) < 3:
            ptrs.append(ctypes.c_void_p(0))
        self._check(self._lib.nufft_setpts(self._h, M, *ptrs))
        self.M = M
        self._pts_keepalive = coords   # the library copies; kept only until the stream passes
        return self

    def setpts_type3(self, X, S):
        """Type 3: sources X (list of d device tensors of M values) and targets S (list of d
        device tensors of K frequencies)."""
        if self.type != 3 or len(X) != self.dim or len(S) != self.dim:
            raise ValueError(f"a type 3 plan in {self.dim}D takes {self.dim} source and target arrays")
        rd = _real_dtype(self.prec)
        M, K = X[0].numel(), S[0].numel()
        xp = [self._dev_tensor(t, rd, M, "x") for t in X] + [ctypes.c_void_p(0)] * (3 - self.dim)
        sp = [self._dev_tensor(t, rd, K, "s") for t in S] + [ctypes.c_void_p(0)] * (3 - self.dim)
        self._check(self._lib.nufft_setpts_type3(self._h, M, *xp, K, *sp))
        self.M, self.K = M, K
        self.n = self.info()["n"]
        return self

    def execute(self, c, f):
        if self.M < 0:
            raise NufftError(NUFFT_ERR_BAD_STATE, "setpts first")
        cd = _complex_dtype(self.prec)
        cp = self._dev_tensor(c, cd, self.M, "c")
        fp = self._dev_tensor(f, cd, self.K if self.type == 3 else self.nmodes, "f")
        self._check(self._lib.nufft_execute(self._h, cp, fp))
        return f if self.type == 1 else c

    def execute_adjoint(self, c, f):
        """The adjoint transform on the same points (type 2 for a type 1 plan, and back)."""
        if self.M < 0:
            raise NufftError(NUFFT_ERR_BAD_STATE, "setpts first")
        cd = _complex_dtype(self.prec)
        cp = self._dev_tensor(c, cd, self.M, "c")
        fp = self._dev_tensor(f, cd, self.nmodes, "f")
        self._check(self._lib.nufft_execute_adjoint(self._h, cp, fp))
        return c if self.type == 1 else f

    def _many(self, fn, c, f):
        if self.M < 0:
            raise NufftError(NUFFT_ERR_BAD_STATE, "setpts first")
        nvec = c.shape[0] if c.dim() > 1 else 1
        if f.shape[0] != nvec or c.dim() != 2 or f.dim() != self.dim + 1:
            raise ValueError("c must be (nvec, M) and f (nvec, N3, N2, N1)-shaped with the same nvec")
        cd = _complex_dtype(self.prec)
        cp = self._dev_tensor(c, cd, nvec * self.M, "c")
        fp = self._dev_tensor(f, cd, nvec * self.nmodes, "f")
        self._check(fn(self._h, nvec, cp, fp))

    def execute_many(self, c, f):
        """nvec transforms of the plan's type on the same points: c (nvec, M), f (nvec, *N
        reversed); type 1 writes f, type 2 writes c."""
        self._many(self._lib.nufft_execute_many, c, f)
        return f if self.type == 1 else c

    def execute_adjoint_many(self, c, f):
        """nvec adjoint transforms on the same points (type 2 for a type 1 plan, and back)."""
        self._many(self._lib.nufft_execute_adjoint_many, c, f)
        return c if self.type == 1 else f

    def spread(self, c, grid):
        cd = _complex_dtype(self.prec)
        self._check(self._lib.nufft_spread(self._h, self._dev_tensor(c, cd, self.M, "c"),
                                           self._dev_tensor(grid, cd, self.fine_cells, "grid")))
        return grid

    def interp(self, grid, c):
        cd = _complex_dtype(self.prec)
        self._check(self._lib.nufft_interp(self._h, self._dev_tensor(grid, cd, self.fine_cells, "grid"),
                                           self._dev_tensor(c, cd, self.M, "c")))
        return c

    def deconvolve(self, fhat, f):
        cd = _complex_dtype(self.prec)
        self._check(self._lib.nufft_deconvolve(self._h, self._dev_tensor(fhat, cd, self.fine_cells, "fhat"),
                                               self._dev_tensor(f, cd, self.nmodes, "f")))
        return f

    def precorrect_pad(self, f, fhat):
        cd = _complex_dtype(self.prec)
        self._check(self._lib.nufft_precorrect_pad(self._h, self._dev_tensor(f, cd, self.nmodes, "f"),
                                                   self._dev_tensor(fhat, cd, self.fine_cells, "fhat")))
        return fhat

    def get_sort(self):
        """(perm, counts, subproblems) as int32 device tensors."""
        torch = _torch()
        info = self.info()
        dev = torch.device("cuda", torch.cuda.current_device())
        perm = torch.empty(max(self.M, 0), dtype=torch.int32, device=dev)
        counts = torch.empty(info["nbins"], dtype=torch.int32, device=dev)
        sub = torch.empty((info["nsubproblems"], 3), dtype=torch.int32, device=dev)
        self._check(self._lib.nufft_get_sort(
            self._h, ctypes.c_void_p(perm.data_ptr() if perm.numel() else 0),
            ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(sub.data_ptr() if sub.numel() else 0)))
        return perm, counts, sub

    def range_errors(self) -> int:
        """Kernel-support starts found outside their padded tile since plan creation (0 when the
        sort and the kernels agree; see nufft_get_range_errors)."""
        v = ctypes.c_int64()
        self._check(self._lib.nufft_get_range_errors(self._h, ctypes.byref(v)))
        return int(v.value)

    def stage_times(self):
        """ms per step (needs timing=True): sort, spread, type-1 FFT, deconvolve, clear,
        interp, type-2 FFT, precorrect+pad, each averaged over the calls since the previous
        read (the last 16 at most; zeros for a direction never run)."""
        ms = (ctypes.c_double * 8)()
        self._check(self._lib.nufft_get_stage_times(self._h, ms))
        keys = ["sort", "spread", "fft1", "deconv", "clear", "interp", "fft2", "pad"]
        return dict(zip(keys, list(ms)))

    def destroy(self):
        if self._h is not None:
            self._lib.nufft_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
