"""Many-vector execution on one setpts (nufft_execute_many / nufft_execute_adjoint_many): every
vector of a batch against the oracle NUFFT, batches split by max_batch, and the argument checks.
Sizes span several bins and subproblems; the batch split leaves a ragged last batch."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from nonuniform_fft_amd.workloads import Workload, make_inputs  # noqa: E402

from _gpu_util import cdtype, dev, to_dev, tol_for  # noqa: E402


@pytest.fixture(scope="module")
def nf():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import nonuniform_fft_amd as nf
    nf.load_library()
    return nf


@pytest.fixture(scope="module")
def orc():
    import oracle.oracle as o
    o._load()
    return o


CASES = [
    Workload("mv", 1, (1000,), 30_001, 1e-6, "f32", seed=81),
    Workload("mv", 1, (777,), 20_000, 1e-12, "f64", seed=87),          # 1D fp64: strengths via perm
    Workload("mv", 2, (48, 40), 20_000, 1e-12, "f64", seed=82),
    Workload("mv", 3, (24, 20, 18), 30_000, 1e-5, "f32", seed=83),      # column-run spreading
    Workload("mv", 3, (20, 16, 12), 10_000, 1e-9, "f64", seed=84),      # fp64 column runs + gather
    Workload("mv", 3, (16, 16, 16), 20_000, 1e-2, "f32", seed=85),      # point-patch spreading
]


def _vectors(wl, nvec, seed):
    rng = np.random.default_rng(seed)
    shape_f = (nvec,) + tuple(reversed(wl.N))
    c = rng.standard_normal((nvec, wl.M)) + 1j * rng.standard_normal((nvec, wl.M))
    f = rng.standard_normal(shape_f) + 1j * rng.standard_normal(shape_f)
    cd = np.complex64 if wl.precision == "f32" else np.complex128
    return c.astype(cd), f.astype(cd)


@pytest.mark.parametrize("wl", CASES, ids=lambda w: f"{w.dim}d_{w.N}_{w.precision}_{w.eps:g}")
@pytest.mark.parametrize("max_batch,method", [(0, 0), (2, 0), (0, 1)], ids=["auto", "batch2", "GMsort"])
def test_many_vectors_vs_oracle(nf, orc, wl, max_batch, method):
    nvec = 5
    print(f"many {wl.N} {wl.precision} eps={wl.eps} nvec={nvec} max_batch={max_batch} method={method}", flush=True)
    sys.stdout.flush()
    X = make_inputs(wl, want_c=False, want_f=False)["X"]
    c, f = _vectors(wl, nvec, 7)
    cd = cdtype(wl.precision)
    p = nf.Plan(1, wl.N, wl.eps, wl.precision, max_batch=max_batch, method=method)
    p.setpts(*[to_dev(x) for x in X])
    f_out = torch.empty((nvec,) + tuple(reversed(wl.N)), dtype=cd, device=dev())
    c_out = torch.empty((nvec, wl.M), dtype=cd, device=dev())
    p.execute_many(to_dev(c), f_out)
    p.execute_adjoint_many(c_out, to_dev(f))
    torch.cuda.synchronize()
    fg, cg = f_out.cpu().numpy(), c_out.cpu().numpy()
    p.destroy()
    tol = tol_for(wl.precision)
    for v in range(nvec):
        e1 = orc.rel_l2(fg[v], orc.nufft_type1(X, c[v], wl.N, wl.eps))
        e2 = orc.rel_l2(cg[v], orc.nufft_type2(X, f[v], wl.N, wl.eps))
        assert e1 <= tol and e2 <= tol, (v, e1, e2)


def test_type2_plan_many_and_single_agree(nf, orc):
    """A type 2 plan: execute_many equals single executes (interpolation is deterministic and the
    batched and single FFTs agree to rounding), and matches the oracle."""
    wl = Workload("mv", 2, (64, 48), 25_000, 1e-5, "f32", seed=86)
    X = make_inputs(wl, want_c=False, want_f=False)["X"]
    nvec = 3
    _, f = _vectors(wl, nvec, 8)
    p = nf.Plan(2, wl.N, wl.eps, wl.precision)
    p.setpts(*[to_dev(x) for x in X])
    cm = torch.empty((nvec, wl.M), dtype=torch.complex64, device=dev())
    p.execute_many(cm, to_dev(f))
    single = []
    for v in range(nvec):
        cv = torch.empty(wl.M, dtype=torch.complex64, device=dev())
        p.execute(cv, to_dev(f[v]))
        single.append(cv)
    torch.cuda.synchronize()
    cm = cm.cpu().numpy()
    for v in range(nvec):
        s = single[v].cpu().numpy()
        assert np.linalg.norm(cm[v] - s) <= 1e-6 * np.linalg.norm(s)
        assert orc.rel_l2(cm[v], orc.nufft_type2(X, f[v], wl.N, wl.eps)) <= tol_for(wl.precision)
    p.destroy()


def test_many_argument_checks(nf):
    import ctypes
    p = nf.Plan(1, (16, 16), 1e-5, "f32")
    p.setpts(to_dev(np.zeros(4, np.float32)), to_dev(np.zeros(4, np.float32)))
    c = torch.ones((2, 4), dtype=torch.complex64, device=dev())
    f = torch.empty((2, 16, 16), dtype=torch.complex64, device=dev())
    lib = nf.load_library()
    assert lib.nufft_execute_many(p.handle, 0, ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(f.data_ptr())) == -1
    assert lib.nufft_execute_many(p.handle, 2, ctypes.c_void_p(c.data_ptr()), None) == -1
    # one vector through the many-vector entry point equals execute
    f1 = torch.empty((1, 16, 16), dtype=torch.complex64, device=dev())
    p.execute_many(c[:1], f1)
    f2 = torch.empty((16, 16), dtype=torch.complex64, device=dev())
    p.execute(c[0], f2)
    torch.cuda.synchronize()
    np.testing.assert_allclose(f1[0].cpu().numpy(), f2.cpu().numpy(), rtol=0, atol=1e-5)
    p.destroy()
