"""nufft_setpts_noalloc (the entry point for callers that cannot allocate) against nufft_setpts,
through the C ABI: on two calls in a row, the second with fewer points, the permutation, bin
counts and subproblem rows are identical to those of nufft_setpts on the same points, and the
transforms run on those points match nufft_setpts's to the parity bars (type 2 bit for bit, type 1
within the rounding of its atomic sums).  No device memory is taken by the calls, sizes past the
scratch or past the plan's buffers are rejected with NUFFT_ERR_ALLOC, and the plan stays usable."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from nonuniform_fft_amd.workloads import Workload, make_inputs  # noqa: E402

from _gpu_util import cdtype, dev, to_dev  # noqa: E402


@pytest.fixture(scope="module")
def nf():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import nonuniform_fft_amd as nf
    nf.load_library()
    return nf


def _ptrs(X):
    p = [ctypes.c_void_p(x.data_ptr()) for x in X]
    return p + [ctypes.c_void_p(0)] * (3 - len(p))


def _sort_state(p):
    perm, counts, sub = p.get_sort()
    return perm.cpu().numpy(), counts.cpu().numpy(), sub.cpu().numpy()


def _pair(p, wl, inp):
    cd = cdtype(wl.precision)
    f = torch.empty(tuple(reversed(wl.N)), dtype=cd, device=dev())
    c = torch.empty(wl.M, dtype=cd, device=dev())
    p.execute(to_dev(inp["c"]), f)
    p.execute_adjoint(c, to_dev(inp["f"]))
    torch.cuda.synchronize()
    return f.cpu().numpy(), c.cpu().numpy()


CASES = [
    ("3d_f32_columns", 3, (24, 20, 18), 40_000, 15_000, 1e-5, "f32", 0),
    ("2d_f64", 2, (64, 48), 30_000, 9_001, 1e-12, "f64", 0),
    ("1d_f32", 1, (3000,), 50_000, 20_000, 1e-6, "f32", 0),
    ("3d_f32_gm", 3, (16, 16, 16), 20_000, 7_000, 1e-5, "f32", 3),
]


@pytest.mark.parametrize("name,dim,N,M1,M2,eps,prec,method", CASES, ids=[c[0] for c in CASES])
def test_setpts_noalloc_matches_setpts(nf, name, dim, N, M1, M2, eps, prec, method):
    lib = nf.load_library()
    print(f"setpts_noalloc {name}", flush=True)
    wl1 = Workload("na", dim, N, M1, eps, prec, seed=301)
    wl2 = Workload("na", dim, N, M2, eps, prec, dist="cluster", seed=302)
    inp1, inp2 = make_inputs(wl1), make_inputs(wl2)
    X1 = [to_dev(x) for x in inp1["X"]]
    X2 = [to_dev(x) for x in inp2["X"]]
    tol1 = 1e-6 if prec == "f32" else 1e-12
    if method == 3:
        tol1 = 1e-5 if prec == "f32" else 1e-12   # every contribution is an atomic in the plan precision

    ref = nf.Plan(1, N, eps, prec, method=method)   # the existing entry point
    nal = nf.Plan(1, N, eps, prec, method=method)   # the no-allocation entry point
    # without an earlier nufft_setpts the plan has no point buffers: rejected, nothing allocated
    rc = lib.nufft_setpts_noalloc(nal.handle, M1, *_ptrs(X1))
    assert rc == nf.NUFFT_ERR_ALLOC, rc
    # size the plan's buffers: the clustered set may need more subproblems, the first more points
    nal.setpts(*X2)
    nal.setpts(*X1)
    # the first call loads the code object that holds the scratch array (once per process and GPU)
    assert lib.nufft_setpts_noalloc(nal.handle, 0, None, None, None) == 0

    for wl, inp, X in ((wl1, inp1, X1), (wl2, inp2, X2)):
        ref.setpts(*X)
        ref_sort = _sort_state(ref)
        f_ref, c_ref = _pair(ref, wl, inp)
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info()[0]
        rc = lib.nufft_setpts_noalloc(nal.handle, wl.M, *_ptrs(X))
        torch.cuda.synchronize()
        free_after = torch.cuda.mem_get_info()[0]
        assert rc == 0, lib.nufft_last_error(nal.handle)
        assert free_after == free_before
        nal.M = wl.M
        got = _sort_state(nal)
        for a, b in zip(got, ref_sort):
            np.testing.assert_array_equal(a, b)
        f, c = _pair(nal, wl, inp)
        np.testing.assert_array_equal(c, c_ref)
        assert np.linalg.norm(f - f_ref) <= tol1 * np.linalg.norm(f_ref)
        assert nal.range_errors() == 0
    # more points than the plan's buffers hold: rejected, the plan keeps no points, and a
    # regular setpts makes it usable again
    big = Workload("na", dim, N, M1 + 1, eps, prec, seed=303)
    Xb = [to_dev(x) for x in make_inputs(big, want_c=False, want_f=False)["X"]]
    assert lib.nufft_setpts_noalloc(nal.handle, big.M, *_ptrs(Xb)) == nf.NUFFT_ERR_ALLOC
    cc = torch.zeros(big.M, dtype=cdtype(prec), device=dev())
    ff = torch.empty(tuple(reversed(N)), dtype=cdtype(prec), device=dev())
    assert lib.nufft_execute(nal.handle, ctypes.c_void_p(cc.data_ptr()), ctypes.c_void_p(ff.data_ptr())) == \
        nf.NUFFT_ERR_BAD_STATE
    nal.setpts(*Xb)
    ref.destroy()
    nal.destroy()


def test_setpts_noalloc_scratch_limit(nf):
    """A point set whose sort needs more than the device scratch array is rejected up front."""
    lib = nf.load_library()
    N = (32, 32, 32)
    p = nf.Plan(1, N, 1e-5, "f32")
    M = 4 << 20          # 3D fp32: about 29 bytes of sort scratch per point, above 64 MiB
    x = torch.zeros(M, dtype=torch.float32, device=dev())
    p.setpts(x, x, x)    # the plan's own buffers can hold M points
    rc = lib.nufft_setpts_noalloc(p.handle, M, *_ptrs([x, x, x]))
    assert rc == nf.NUFFT_ERR_ALLOC
    assert b"scratch" in lib.nufft_last_error(p.handle)
    p.destroy()
