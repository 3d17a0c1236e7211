"""Full-size parity: every benchmark configuration at its real size, run through the C ABI in
the launch configuration the benchmark times (one plan: setpts, type 1, adjoint type 2).

The oracle cannot form these transforms whole in seconds, so outputs are compared on samples
it computes one by one:
  * type 1: chosen modes, by eq. (9) at those frequencies with eq. (7) inserted (the oracle's
    type1_at) -- the same approximation as the library, to 1e-5 (fp32) / 1e-10 (fp64);
  * type 2: chosen points, interpolated from the oracle's full fine grid (eqs. (11), (12));
  * both against the exact sums (eqs. (1), (3)) at a few outputs, within 10 eps.
"""
import sys

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
    ("2d_n1024_m4m_f32_e5", 48, 48),
    ("2d_n1024_m4m_f64_e12", 24, 48),
    ("3d_n128_m16m_f32_e2", 32, 48),
    ("3d_n128_m16m_f32_e5", 24, 48),
    ("3d_n128_m16m_f32_e5_cluster", 24, 48),
    ("3d_n256_m134m_f64_e9", 8, 24),
    ("1d_n1m_m16m_f32_e6", 48, 48),
    ("1d_n1m_m16m_f64_e6", 48, 48),
]


@pytest.mark.parametrize("name,nmodes,npts", CONFIGS, ids=[c[0] for c in CONFIGS])
def test_full_size_config(nf, orc, name, nmodes, npts):
    wl = WORKLOADS[name]
    print(f"full-size {name}: N={wl.N} M={wl.M} {wl.precision} eps={wl.eps} {wl.dist}", flush=True)
    sys.stdout.flush()
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
    f_gpu = f_out.cpu().numpy().ravel()
    c_gpu = c_out.cpu().numpy()
    del Xd, c_d, f_d, f_out, c_out
    plan.destroy()
    torch.cuda.empty_cache()

    rng = np.random.default_rng(7)
    sel_k = _sample_modes(wl.N, nmodes, rng)
    sel_j = _sample_points(wl.M, npts, rng)
    tol = tol_for(wl.precision)

    # type 1 at chosen modes vs the oracle's same approximation
    ref1 = orc.nufft_type1_at(X, c, wl.N, wl.eps, sel_k)
    e1 = orc.rel_l2(f_gpu[sel_k], ref1)
    print(f"  type1 vs oracle at {len(sel_k)} modes: {e1:.2e}", flush=True)
    assert e1 <= tol, e1

    # type 2 at chosen points vs the oracle's fine grid
    ref2 = orc.nufft_type2_at(X, f, wl.N, wl.eps, sel_j)
    e2 = orc.rel_l2(c_gpu[sel_j], ref2)
    print(f"  type2 vs oracle at {len(sel_j)} points: {e2:.2e}", flush=True)
    assert e2 <= tol, e2

    # a few outputs against the exact sums, within 10 eps
    kk = sel_k[:4]
    jj = sel_j[:4]
    d1 = orc.rel_l2(f_gpu[kk], orc.direct_type1(X, c, wl.N, sel=kk))
    d2 = orc.rel_l2(c_gpu[jj], orc.direct_type2(X, f, wl.N, sel=jj))
    print(f"  vs exact sums: type1 {d1:.2e}  type2 {d2:.2e}  (10 eps = {10 * wl.eps:g})", flush=True)
    assert d1 <= 10 * wl.eps and d2 <= 10 * wl.eps
