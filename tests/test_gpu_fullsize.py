"""Full-size parity: every benchmark configuration at its real size, run through the C ABI in
the launch configuration the benchmark times (one plan: setpts, type 1, adjoint type 2).

Whole outputs are compared with the oracle NUFFT (eqs. (7)-(12), relative l2 over all modes and
all points, cuFINUFFT page Sec. IV-C) for every configuration whose oracle grid fits in seconds:
the oracle's spreading and interpolation run in their parallel forms, which equal the serial
loops bit for bit.  The 256^3 fp64 configuration (2^27 points, w = 10: 1.3e11 cell updates per
transform) is compared on samples the oracle computes one by one:
  * type 1: chosen modes, by eq. (9) at those frequencies with eq. (7) inserted (the oracle's
    type1_at) -- the same approximation as the library;
  * type 2: 4096 chosen points, interpolated from the oracle's full fine grid (eqs. (11), (12)).
Every configuration is also checked against the exact sums (eqs. (1), (3)) at a few outputs,
within 10 eps.
"""
import sys
import time

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from nonuniform_fft_amd.workloads import WORKLOADS, make_inputs  # noqa: E402

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


def _sample_modes(N, count, rng):
    """Flat output positions (k1 fastest): the corners of I_N, k = 0, and random modes."""
    total = int(np.prod(N))
    picks = {0, total - 1}
    center = 0
    for i, Ni in reversed(list(enumerate(N))):
        center = center * Ni + Ni // 2
    picks.add(center)
    while len(picks) < count:
        picks.add(int(rng.integers(0, total)))
    return np.array(sorted(picks), dtype=np.int64)


def _sample_points(M, count, rng):
    picks = {0, M - 1}
    while len(picks) < count:
        picks.add(int(rng.integers(0, M)))
    return np.array(sorted(picks), dtype=np.int64)


CONFIGS = [
    # name, whole outputs?, sampled modes, sampled points
    ("2d_n1024_m4m_f32_e5", True, 0, 0),
    ("2d_n1024_m4m_f64_e12", True, 0, 0),
    ("3d_n128_m16m_f32_e2", True, 0, 0),
    ("3d_n128_m16m_f32_e5", True, 0, 0),
    ("3d_n128_m16m_f32_e5_cluster", True, 0, 0),
    ("3d_n256_m134m_f64_e9", False, 12, 4096),
    ("1d_n1m_m16m_f32_e6", True, 0, 0),
    ("1d_n1m_m16m_f64_e6", True, 0, 0),
]


@pytest.mark.parametrize("name,whole,nmodes,npts", CONFIGS, ids=[c[0] for c in CONFIGS])
def test_full_size_config(nf, orc, name, whole, nmodes, npts):
    wl = WORKLOADS[name]
    print(f"full-size {name}: N={wl.N} M={wl.M} {wl.precision} eps={wl.eps} {wl.dist}", flush=True)
    sys.stdout.flush()
    t0 = time.perf_counter()
    inp = make_inputs(wl)
    X, c, f = inp["X"], inp["c"], inp["f"]
    cd = cdtype(wl.precision)
    plan = nf.Plan(1, wl.N, wl.eps, wl.precision)
    Xd = [to_dev(x) for x in X]
    plan.setpts(*Xd)
    c_d = to_dev(c)
    f_d = to_dev(f)
    f_out = torch.empty(tuple(reversed(wl.N)), dtype=cd, device=dev())
    c_out = torch.empty(wl.M, dtype=cd, device=dev())
    plan.execute(c_d, f_out)
    plan.execute_adjoint(c_out, f_d)
    torch.cuda.synchronize()
    assert plan.range_errors() == 0
    f_gpu = f_out.cpu().numpy().ravel()
    c_gpu = c_out.cpu().numpy()
    del Xd, c_d, f_d, f_out, c_out
    plan.destroy()
    torch.cuda.empty_cache()
    print(f"  inputs + GPU pair: {time.perf_counter() - t0:.1f} s", flush=True)
    tol = tol_for(wl.precision)
    rng = np.random.default_rng(7)

    if whole:
        t1 = time.perf_counter()
        ref1 = orc.nufft_type1(X, c, wl.N, wl.eps).ravel()
        e1 = orc.rel_l2(f_gpu, ref1)
        print(f"  type1 vs oracle, all {f_gpu.size} modes: {e1:.2e} ({time.perf_counter() - t1:.1f} s)", flush=True)
        del ref1
        t1 = time.perf_counter()
        ref2 = orc.nufft_type2(X, f, wl.N, wl.eps)
        e2 = orc.rel_l2(c_gpu, ref2)
        print(f"  type2 vs oracle, all {c_gpu.size} points: {e2:.2e} ({time.perf_counter() - t1:.1f} s)", flush=True)
        del ref2
        sel_k = _sample_modes(wl.N, 4, rng)
        sel_j = _sample_points(wl.M, 4, rng)
    else:
        sel_k = _sample_modes(wl.N, nmodes, rng)
        sel_j = _sample_points(wl.M, npts, rng)
        t1 = time.perf_counter()
        ref1 = orc.nufft_type1_at(X, c, wl.N, wl.eps, sel_k)
        e1 = orc.rel_l2(f_gpu[sel_k], ref1)
        print(f"  type1 vs oracle at {len(sel_k)} modes: {e1:.2e} ({time.perf_counter() - t1:.1f} s)", flush=True)
        t1 = time.perf_counter()
        ref2 = orc.nufft_type2_at(X, f, wl.N, wl.eps, sel_j)
        e2 = orc.rel_l2(c_gpu[sel_j], ref2)
        print(f"  type2 vs oracle at {len(sel_j)} points: {e2:.2e} ({time.perf_counter() - t1:.1f} s)", flush=True)
    assert e1 <= tol, e1
    assert e2 <= tol, e2

    # a few outputs against the exact sums, within 10 eps
    kk = sel_k[:4]
    jj = sel_j[:4]
    d1 = orc.rel_l2(f_gpu[kk], orc.direct_type1(X, c, wl.N, sel=kk))
    d2 = orc.rel_l2(c_gpu[jj], orc.direct_type2(X, f, wl.N, sel=jj))
    print(f"  vs exact sums: type1 {d1:.2e}  type2 {d2:.2e}  (10 eps = {10 * wl.eps:g})", flush=True)
    assert d1 <= 10 * wl.eps and d2 <= 10 * wl.eps


def test_fine_grid_above_2_31_cells(nf, orc):
    """The largest grid class a plan accepts: 3D fp32 with N = 1024 x 1024 x 500 modes on a
    2048 x 2048 x 1000 fine grid, 4.19e9 cells (above 2^31, below the 2^32 limit; two 31 GiB grid
    buffers), so every linear cell index exceeds a signed 32-bit integer somewhere in the grid.
    Type 1 at 64 modes and type 2 at all points are compared with the exact sums (eqs. (1), (3))
    within 10 eps; the type 2 coefficients have 16 nonzero modes, so their exact sum is cheap."""
    from nonuniform_fft_amd.workloads import Workload
    N = (1024, 1024, 500)
    wl = Workload("grid_big", 3, N, 4096, 1e-5, "f32", seed=171)
    print(f"largest grid: N={N} M={wl.M}", flush=True)
    inp = make_inputs(wl, sparse_f=16)
    X, c = inp["X"], inp["c"]
    plan = nf.Plan(1, N, wl.eps, "f32")
    assert tuple(plan.info()["n"][:3]) == (2048, 2048, 1000)
    plan.setpts(*[to_dev(x) for x in X])
    f_out = torch.empty(tuple(reversed(N)), dtype=torch.complex64, device=dev())
    plan.execute(to_dev(c), f_out)
    f_in = torch.zeros(tuple(reversed(N)), dtype=torch.complex64, device=dev())
    f_in.view(-1)[torch.from_numpy(inp["f_modes"]).to(dev())] = to_dev(inp["f_vals"])
    c_out = torch.empty(wl.M, dtype=torch.complex64, device=dev())
    plan.execute_adjoint(c_out, f_in)
    torch.cuda.synchronize()
    assert plan.range_errors() == 0
    rng = np.random.default_rng(9)
    sel_k = _sample_modes(N, 64, rng)
    f_sel = f_out.view(-1)[torch.from_numpy(sel_k).to(dev())].cpu().numpy()
    c_gpu = c_out.cpu().numpy()
    del f_out, f_in, c_out
    plan.destroy()
    torch.cuda.empty_cache()
    d1 = orc.rel_l2(f_sel, orc.direct_type1(X, c, N, sel=sel_k))
    d2 = orc.rel_l2(c_gpu, orc.direct_type2_modes(X, N, inp["f_modes"], inp["f_vals"]))
    print(f"  vs exact sums: type1 at 64 modes {d1:.2e}, type2 at all points {d2:.2e}", flush=True)
    assert d1 <= 10 * wl.eps and d2 <= 10 * wl.eps
