"""Status codes that need a device: the allocation cap (opts.max_device_bytes -> NUFFT_ERR_ALLOC)
and the tolerance clamp (NUFFT_WARN_EPS_CLAMPED), through the C ABI."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from _gpu_util import cdtype, dev, to_dev  # noqa: E402


@pytest.fixture(scope="module")
def nf():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import nonuniform_fft_amd as nf
    nf.load_library()
    return nf


def _create(lib, nf, t, N, eps, prec, **fields):
    from nonuniform_fft_amd._native import NufftOpts
    o = NufftOpts()
    lib.nufft_default_opts(ctypes.byref(o))
    for k, v in fields.items():
        setattr(o, k, v)
    Narr = (ctypes.c_int64 * len(N))(*N)
    h = ctypes.c_void_p()
    rc = lib.nufft_plan_create(t, len(N), Narr, eps, prec, None, ctypes.byref(o), ctypes.byref(h))
    return rc, h


def test_alloc_cap_at_plan_create(nf):
    """A cap below the fine grid's size fails plan creation with NUFFT_ERR_ALLOC and no plan."""
    lib = nf.load_library()
    rc, h = _create(lib, nf, 1, (64, 64), 1e-5, 0, max_device_bytes=1000)
    assert rc == nf.NUFFT_ERR_ALLOC
    assert not h.value


def test_alloc_cap_at_setpts_keeps_plan_usable(nf):
    """A cap that admits the plan but not the sort buffers of many points fails setpts with
    NUFFT_ERR_ALLOC; the plan keeps no points (execute is a state error) and still takes a
    smaller point set."""
    lib = nf.load_library()
    N = (32, 32)
    # fine grid 64^2 x 8 B, correction factors, FFT work: well under 1 MB; 2^20 points need
    # more than 20 MB of sort buffers
    rc, h = _create(lib, nf, 1, N, 1e-5, 0, max_device_bytes=1 << 20)
    assert rc == 0 and h.value
    try:
        M = 1 << 20
        x = torch.zeros(M, dtype=torch.float32, device=dev())
        rc = lib.nufft_setpts(h, M, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()), None)
        assert rc == nf.NUFFT_ERR_ALLOC
        assert b"max_device_bytes" in lib.nufft_last_error(h)
        c = torch.ones(M, dtype=torch.complex64, device=dev())
        f = torch.empty((32, 32), dtype=torch.complex64, device=dev())
        assert lib.nufft_execute(h, ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(f.data_ptr())) == nf.NUFFT_ERR_BAD_STATE
        # a small point set fits under the cap: one point at the origin gives f_k = 1
        x1 = torch.zeros(1, dtype=torch.float32, device=dev())
        assert lib.nufft_setpts(h, 1, ctypes.c_void_p(x1.data_ptr()), ctypes.c_void_p(x1.data_ptr()), None) == 0
        assert lib.nufft_execute(h, ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(f.data_ptr())) == 0
        torch.cuda.synchronize()
        assert torch.allclose(f, torch.ones_like(f), atol=1e-4)
    finally:
        lib.nufft_destroy(h)


@pytest.mark.parametrize("eps,w_expect", [(1e-20, 16), (2.0, 2), (10.0, 2)])
def test_eps_clamp_warning(nf, eps, w_expect):
    """eps asking for a width outside [2, 16] returns NUFFT_WARN_EPS_CLAMPED with w clamped, and
    the plan works (a single point at x = 0.5 gives f_k = exp(-i k 0.5) within the clamped
    kernel's accuracy)."""
    p = nf.Plan(1, (40,), eps, "f64")
    assert p.warning == nf.NUFFT_WARN_EPS_CLAMPED
    assert p.w == w_expect
    p.setpts(to_dev(np.array([0.5])))
    f = torch.empty(40, dtype=cdtype("f64"), device=dev())
    p.execute(torch.ones(1, dtype=cdtype("f64"), device=dev()), f)
    torch.cuda.synchronize()
    k = np.arange(-20, 20)
    exact = np.exp(-1j * k * 0.5)
    err = np.linalg.norm(f.cpu().numpy() - exact) / np.linalg.norm(exact)
    assert err <= (1e-13 if w_expect == 16 else 0.5), err
    p.destroy()
    # a width inside the range gives no warning
    q = nf.Plan(1, (40,), 1e-6, "f64")
    assert q.warning == 0 and q.w == 7
    q.destroy()
