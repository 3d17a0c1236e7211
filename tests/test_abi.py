"""Host-only checks of the C ABI: the library loads, exports every declared entry point, and
rejects invalid arguments before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nufft_amd.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nufft_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("nufft_plan_create", "nufft_setpts", "nufft_execute", "nufft_destroy"):
        assert required in names


def test_library_exports_every_declared_symbol():
    import nonuniform_fft_amd as nf
    lib = nf.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    # and the binding knows every one of them
    from nonuniform_fft_amd._native import SIGNATURES
    assert set(SIGNATURES) == set(_declared_functions())


def test_host_side_argument_checks():
    import nonuniform_fft_amd as nf
    from nonuniform_fft_amd._native import NufftOpts
    lib = nf.load_library()
    assert lib.nufft_default_opts(None) == -1
    o = NufftOpts()
    assert lib.nufft_default_opts(ctypes.byref(o)) == 0 and o.method == 0
    assert lib.nufft_destroy(None) == 0
    N = (ctypes.c_int64 * 3)(16, 16, 16)
    h = ctypes.c_void_p()
    bad = [(4, 2, N, 1e-5, 0), (0, 2, N, 1e-5, 0), (1, 4, N, 1e-5, 0), (1, 0, N, 1e-5, 0), (1, 2, N, 0.0, 0), (1, 2, N, -1.0, 0),
           (1, 2, N, float("nan"), 0), (1, 2, N, 1e-5, 2), (1, 2, None, 1e-5, 0),
           (2, 3, (ctypes.c_int64 * 3)(16, 0, 16), 1e-5, 1),
           # a mode count above 2^28, and fine grids of 2^32 and 2^38 cells
           (1, 1, (ctypes.c_int64 * 3)((1 << 28) + 1, 1, 1), 1e-5, 0),
           (1, 3, (ctypes.c_int64 * 3)(1 << 10, 1 << 10, 1 << 9), 1e-5, 0),
           (1, 3, (ctypes.c_int64 * 3)(1 << 12, 1 << 12, 1 << 11), 1e-5, 0)]
    for t, d, n, e, p in bad:
        assert lib.nufft_plan_create(t, d, n, e, p, None, None, ctypes.byref(h)) == -1
        assert not h.value
    assert lib.nufft_plan_create(1, 2, N, 1e-5, 0, None, None, None) == -1
    # type 3 supports sigma = 2 only
    o = NufftOpts()
    lib.nufft_default_opts(ctypes.byref(o))
    o.upsampfac = 1.5
    assert lib.nufft_plan_create(3, 2, None, 1e-5, 0, None, ctypes.byref(o), ctypes.byref(h)) == -7
    assert not h.value
    # an upsampling factor outside [1.25, 2] is rejected before any device work
    for sigma in (1.1, 2.5, -1.0, float("nan")):
        o = NufftOpts()
        lib.nufft_default_opts(ctypes.byref(o))
        o.upsampfac = sigma
        assert lib.nufft_plan_create(1, 2, N, 1e-5, 0, None, ctypes.byref(o), ctypes.byref(h)) == -1
        assert not h.value
    for code in (0, 1, -1, -2, -3, -4, -5, -6, -7):
        assert lib.nufft_strerror(code)
    assert lib.nufft_strerror(12345) == b"unknown status"
    for fn in ("nufft_setpts", "nufft_execute", "nufft_spread", "nufft_interp"):
        args = {"nufft_setpts": (None, 0, None, None, None)}.get(fn, (None, None, None))
        assert getattr(lib, fn)(*args) == -1


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from nonuniform_fft_amd import _native
    monkeypatch.setattr(_native, "_lib", None)
    monkeypatch.setattr(_native, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError):
        _native.load_library()
