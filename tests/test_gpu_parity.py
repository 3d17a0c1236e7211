"""GPU parity tests: the HIP path through the C ABI against the CPU oracle, element by element.

Sizes are chosen so the oracle finishes in seconds while the GPU path still spans several bins
(tiles), several subproblems per bin where forced, and ragged tails in M and in the grid.
"""
import math
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from nonuniform_fft_amd.workloads import WORKLOADS, Workload, make_inputs, scaled  # noqa: E402

from _gpu_util import cdtype, dev, gpu_type1, gpu_type2, to_dev, tol_for  # noqa: E402


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


def _announce(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------------------------------------
# Bin-sort: bit-exact
# ---------------------------------------------------------------------------------------------

SORT_CASES = [
    ("2d_uniform_f32", Workload("s", 2, (100, 72), 50_001, 1e-5, "f32", seed=21)),
    ("2d_uniform_f64", Workload("s", 2, (64, 64), 30_000, 1e-12, "f64", seed=22)),
    ("3d_uniform_f32", Workload("s", 3, (24, 20, 18), 40_000, 1e-5, "f32", seed=23)),
    ("3d_cluster_f32", Workload("s", 3, (32, 32, 32), 60_000, 1e-5, "f32", dist="cluster", seed=24)),
    ("3d_box_f64", Workload("s", 3, (16, 16, 16), 20_000, 1e-9, "f64", dist="box", seed=25)),
    ("2d_tiny", Workload("s", 2, (5, 7), 3, 1e-3, "f32", seed=26)),
    ("1d_uniform_f32", Workload("s", 1, (1000,), 50_001, 1e-5, "f32", seed=27)),
    ("1d_cluster_f64", Workload("s", 1, (777,), 30_000, 1e-12, "f64", dist="cluster", seed=28)),
    ("1d_large_f32", Workload("s", 1, (1 << 16,), 200_000, 1e-6, "f32", seed=29)),
]


def _grid_t(x, n):
    """t = (x + pi) n / (2 pi) in fp64 as two rounded operations, folded once into [0, n) (the
    documented coordinate rule of nufft_get_sort); returns (t, l)."""
    s = np.float64(n) / (2.0 * np.float64(math.pi))
    t = (np.asarray(x, dtype=np.float64) + np.float64(math.pi)) * s
    l = np.floor(t)
    hi, lo = l >= n, l < 0
    t = np.where(hi, t - n, np.where(lo, t + n, t))
    l = np.where(hi, l - n, np.where(lo, l + n, l))
    return t, l.astype(np.int64)


def _documented_inbin_key(X, info):
    """The in-bin key nufft_get_sort documents for plans with a column order (w, s): the block
    (c2 // s) ceil((m1 + 1) / s) + c1 // s of the support start c_i = ceil(t_i - w/2) - (b_i m_i -
    floor(w/2)), then the z start c3.  Computed here from the header's description alone."""
    w, step = info["colw"], info["colstep"]
    m, n = info["bins"], info["n"]
    c = []
    for i in range(3):
        t, l = _grid_t(X[i], n[i])
        b = l // m[i]
        c.append(np.ceil(t - 0.5 * w).astype(np.int64) - (b * m[i] - w // 2))
    ncx = -(-(m[0] + 1) // step)
    return ((c[1] // step) * ncx + c[0] // step) * (m[2] + 1) + c[2]


def _check_sort(info, X, perm, counts, sub, orc):
    """Counts and subproblem rows bit-exact against the oracle; every bin's slice of the
    permutation holds exactly the oracle's points of that bin; the order inside a bin is the
    documented one (increasing original index, or for column-order plans the documented key then
    the original index).  Several in-bin orders are valid; the oracle fixes only the set."""
    _, ocounts, operm = orc.binsort(X, info["n"], info["bins"])
    np.testing.assert_array_equal(counts, ocounts)
    osub = orc.subproblems(ocounts, info["cap"])
    np.testing.assert_array_equal(sub, osub)
    off = np.concatenate([[0], np.cumsum(ocounts)])
    assert perm.size == operm.size
    for b in np.nonzero(ocounts)[0]:
        a, e = off[b], off[b + 1]
        np.testing.assert_array_equal(np.sort(perm[a:e]), operm[a:e])
    # in-bin order
    if info["colw"] > 0:
        key = _documented_inbin_key(X, info)[perm]
    else:
        key = np.zeros(perm.size, dtype=np.int64)
    binpos = np.repeat(np.arange(ocounts.size), ocounts)
    order = np.lexsort((perm, key, binpos))
    np.testing.assert_array_equal(order, np.arange(perm.size))


@pytest.mark.parametrize("name,wl", SORT_CASES, ids=[c[0] for c in SORT_CASES])
@pytest.mark.parametrize("cap", [0, 37])
def test_binsort_bit_exact(nf, orc, name, wl, cap):
    _announce(f"binsort {name} cap={cap}")
    inp = make_inputs(wl, want_f=False)
    X = inp["X"]
    p = nf.Plan(1, wl.N, wl.eps, wl.precision, subproblem_cap=cap)
    p.setpts(*[to_dev(x) for x in X])
    info = p.info()
    perm, counts, sub = [t.cpu().numpy().astype(np.int64) for t in p.get_sort()]
    if cap > 0:
        assert info["cap"] == cap
    _check_sort(info, X, perm, counts, sub, orc)
    p.destroy()


def test_binsort_boundary_points(nf, orc):
    """Coordinates at -pi, just below pi, values that round to pi in fp32, the fold range
    [-3 pi, -pi) and [pi, 3 pi), and nextafter(-pi, -inf), whose folded t rounds to n."""
    N = (32, 24)
    xs = np.array([-math.pi, np.nextafter(math.pi, 0), math.pi - 1e-9, 0.0, 1e-30, -1e-30,
                   -2.9 * math.pi, 2.5 * math.pi, math.pi, -math.pi + 1e-7, np.nextafter(-math.pi, -4.0),
                   3 * math.pi - 1e-5, -3 * math.pi + 1e-5])
    ys = np.array([0.1, -0.2, math.pi - 1e-12, -math.pi, 3.0, -3.0, 0.0, 0.0, 1.0, 2.9, 0.5, -1.5,
                   np.nextafter(-math.pi, -4.0)])
    for prec, dt in (("f32", np.float32), ("f64", np.float64)):
        for N3 in (None, 20):
            X = [xs.astype(dt), ys.astype(dt)]
            NN = N if N3 is None else N + (N3,)
            if N3 is not None:
                X.append(np.roll(xs, 3).astype(dt))
            p = nf.Plan(1, NN, 1e-6, prec)
            p.setpts(*[to_dev(x) for x in X])
            info = p.info()
            perm, counts, sub = [t.cpu().numpy().astype(np.int64) for t in p.get_sort()]
            _check_sort(info, X, perm, counts, sub, orc)
            # the points at the period's ends (folded t rounding onto n) keep their stencils
            # inside their tiles in both directions
            cd = cdtype(prec)
            f = torch.empty(tuple(reversed(NN)), dtype=cd, device=dev())
            cc = torch.empty(len(xs), dtype=cd, device=dev())
            p.execute(torch.ones(len(xs), dtype=cd, device=dev()), f)
            p.execute_adjoint(cc, f)
            torch.cuda.synchronize()
            assert p.range_errors() == 0
            p.destroy()


def test_setpts_rejects_bad_points(nf):
    p = nf.Plan(1, (16, 16), 1e-5, "f32")
    # -3 pi itself scales to t = -n minus a rounding, below the accepted floor(t) >= -n
    for bad in (np.nan, np.inf, 20.0, -10.0, -3 * math.pi):
        x = np.array([0.0, bad, 1.0], np.float32)
        y = np.zeros(3, np.float32)
        with pytest.raises(nf.NufftError) as ei:
            p.setpts(to_dev(x), to_dev(y))
        assert ei.value.code == -6
    # the plan stays usable
    p.setpts(to_dev(np.zeros(3, np.float32)), to_dev(np.zeros(3, np.float32)))
    c = torch.ones(3, dtype=torch.complex64, device=dev())
    f = torch.empty((16, 16), dtype=torch.complex64, device=dev())
    p.execute(c, f)
    torch.cuda.synchronize()
    p.destroy()


def test_execute_before_setpts_is_state_error(nf):
    p = nf.Plan(1, (16, 16), 1e-5, "f32")
    c = torch.ones(3, dtype=torch.complex64, device=dev())
    f = torch.empty((16, 16), dtype=torch.complex64, device=dev())
    p.M = 3  # bypass the Python-side check to reach the C ABI
    with pytest.raises(nf.NufftError) as ei:
        p.execute(c, f)
    assert ei.value.code == -2
    p.destroy()


# ---------------------------------------------------------------------------------------------
# Single steps
# ---------------------------------------------------------------------------------------------

STEP_CASES = [
    Workload("st", 2, (100, 72), 50_001, 1e-5, "f32", seed=31),
    Workload("st", 2, (64, 48), 20_000, 1e-12, "f64", seed=32),
    Workload("st", 3, (24, 20, 18), 40_000, 1e-5, "f32", seed=33),
    Workload("st", 3, (16, 16, 16), 20_000, 1e-2, "f32", seed=34),
    Workload("st", 3, (20, 16, 12), 15_000, 1e-9, "f64", seed=35),
    Workload("st", 3, (16, 16, 16), 30_000, 1e-5, "f32", dist="box", seed=36),
    # fp64 3D box: one bin split into subproblems of the full cap, each interpolated in two
    # chunks of the bank-aware point order
    Workload("st", 3, (16, 16, 16), 30_000, 1e-9, "f64", dist="box", seed=40),
    Workload("st", 1, (1000,), 50_001, 1e-5, "f32", seed=37),
    Workload("st", 1, (777,), 30_000, 1e-12, "f64", seed=38),
    Workload("st", 1, (4096,), 40_000, 1e-6, "f32", dist="box", seed=39),
    # fine grids smaller than one padded bin, which then wraps onto the grid more than once
    Workload("st", 3, (3, 4, 2), 2_000, 1e-5, "f32", seed=131),
    Workload("st", 3, (4, 3, 5), 2_000, 1e-2, "f32", seed=132),
    Workload("st", 3, (4, 4, 4), 1_000, 1e-9, "f64", seed=133),
    Workload("st", 2, (5, 7), 2_000, 1e-12, "f64", seed=134),
    Workload("st", 1, (5,), 2_000, 1e-6, "f32", seed=135),
]


def _step_tol(prec, fp32_atomics=False):
    """Single-step bars.  fp32 kernel weights and one fp32 rounding per output give ~1e-7; the
    GM-sort spread adds every contribution with an fp32 global atomic, whose rounding error grows
    like sqrt(contributions per cell) * 2^-24 (~1e-5 for thousands of points per cell)."""
    if prec == "f64":
        return 1e-12
    return 1e-5 if fp32_atomics else 1e-6


@pytest.mark.parametrize("wl", STEP_CASES, ids=lambda w: f"{w.dim}d_{w.N}_{w.precision}_{w.eps:g}_{w.dist}")
@pytest.mark.parametrize("method", [2, 1, 3], ids=["SM", "GMsort", "GM"])
def test_spread_step(nf, orc, wl, method):
    _announce(f"spread {wl.N} {wl.precision} eps={wl.eps} {wl.dist} method={method}")
    inp = make_inputs(wl, want_f=False)
    p = nf.Plan(1, wl.N, wl.eps, wl.precision, method=method, subproblem_cap=500 if wl.dist == "box" else 0)
    p.setpts(*[to_dev(x) for x in inp["X"]])
    grid = torch.empty(p.fine_cells, dtype=cdtype(wl.precision), device=dev())
    p.spread(to_dev(inp["c"]), grid)
    torch.cuda.synchronize()
    ref = orc.spread(inp["X"], inp["c"], p.n, p.w, p.beta)
    err = orc.rel_l2(grid.cpu().numpy(), ref.ravel())
    assert err <= _step_tol(wl.precision, fp32_atomics=(method in (1, 3))), err
    assert p.range_errors() == 0
    p.destroy()


@pytest.mark.parametrize("wl", STEP_CASES, ids=lambda w: f"{w.dim}d_{w.N}_{w.precision}_{w.eps:g}_{w.dist}")
@pytest.mark.parametrize("method", [2, 1, 3], ids=["SM", "GMsort", "GM"])
def test_interp_step(nf, orc, wl, method):
    _announce(f"interp {wl.N} {wl.precision} eps={wl.eps} {wl.dist} method={method}")
    inp = make_inputs(wl, want_f=False)
    p = nf.Plan(2, wl.N, wl.eps, wl.precision, method=method, subproblem_cap=500 if wl.dist == "box" else 0)
    p.setpts(*[to_dev(x) for x in inp["X"]])
    rng = np.random.default_rng(99)
    g = (rng.standard_normal(p.fine_cells) + 1j * rng.standard_normal(p.fine_cells)).astype(
        np.complex64 if wl.precision == "f32" else np.complex128)
    c = torch.empty(wl.M, dtype=cdtype(wl.precision), device=dev())
    p.interp(to_dev(g), c)
    torch.cuda.synchronize()
    ref = orc.interp(inp["X"], g.reshape(tuple(reversed(p.n))), p.w, p.beta)
    err = orc.rel_l2(c.cpu().numpy(), ref)
    assert err <= _step_tol(wl.precision), err
    assert p.range_errors() == 0
    p.destroy()


@pytest.mark.parametrize("N,prec", [((100, 72), "f32"), ((33, 17), "f64"), ((24, 20, 18), "f32"),
                                    ((9, 16, 7), "f64"), ((1000,), "f32"), ((777,), "f64")])
def test_correction_steps(nf, orc, N, prec):
    eps = 1e-5 if prec == "f32" else 1e-11
    prm = orc.Params(N, eps)
    rng = np.random.default_rng(5)
    cd = np.complex64 if prec == "f32" else np.complex128
    # type 1 step 3
    p1 = nf.Plan(1, N, eps, prec)
    fhat = (rng.standard_normal(tuple(reversed(prm.n))) + 1j * rng.standard_normal(tuple(reversed(prm.n)))).astype(cd)
    f = torch.empty(tuple(reversed(N)), dtype=cdtype(prec), device=dev())
    p1.deconvolve(to_dev(fhat), f)
    torch.cuda.synchronize()
    ref = orc.truncate_correct(fhat.astype(np.complex128), prm)
    assert orc.rel_l2(f.cpu().numpy(), ref) <= (1e-6 if prec == "f32" else 1e-13)
    p1.destroy()
    # type 2 step 1
    p2 = nf.Plan(2, N, eps, prec)
    fin = (rng.standard_normal(tuple(reversed(N))) + 1j * rng.standard_normal(tuple(reversed(N)))).astype(cd)
    out = torch.full((int(np.prod(prm.n)),), 7.0, dtype=cdtype(prec), device=dev())
    p2.precorrect_pad(to_dev(fin), out)
    torch.cuda.synchronize()
    ref2 = orc.precorrect_pad(fin.astype(np.complex128), prm)
    assert orc.rel_l2(out.cpu().numpy(), ref2.ravel()) <= (1e-6 if prec == "f32" else 1e-13)
    p2.destroy()


@pytest.mark.parametrize("N,sigma", [((100, 72), 2.0), ((24, 20, 18), 2.0), ((1000,), 2.0),
                                     ((37, 22, 9), 1.25), ((60, 20), 1.25), ((60, 20, 8), 1.25)])
def test_precorrect_pad_store_paths(nf, orc, N, sigma):
    """fp32 pre-correction into a 16-byte-aligned grid with an even first fine size writes two cells per
    thread; an output 8 bytes off alignment (or an odd first fine size) writes one.  Both must give
    the same values, zero every cell outside the modes, and match the oracle's padding step."""
    prm = orc.Params(N, 1e-5, sigma=sigma)
    p = nf.Plan(2, N, 1e-5, "f32", upsampfac=sigma if sigma != 2.0 else 0.0)
    assert tuple(p.n) == prm.n
    total = int(np.prod(prm.n))
    rng = np.random.default_rng(11)
    fin = (rng.standard_normal(tuple(reversed(N))) + 1j * rng.standard_normal(tuple(reversed(N)))).astype(np.complex64)
    fd = to_dev(fin)
    buf_a = torch.full((total + 1,), 7.0, dtype=torch.complex64, device=dev())
    buf_b = torch.full((total + 1,), 7.0, dtype=torch.complex64, device=dev())
    out_a, out_b = buf_a[:total], buf_b[1:]
    assert out_a.data_ptr() % 16 == 0 and out_b.data_ptr() % 16 == 8
    p.precorrect_pad(fd, out_a)
    p.precorrect_pad(fd, out_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert buf_a[total].item() == 7.0 and buf_b[0].item() == 7.0
    ref = orc.precorrect_pad(fin.astype(np.complex128), prm).ravel()
    got = out_a.cpu().numpy()
    assert np.all(got[ref == 0] == 0)
    assert orc.rel_l2(got, ref) <= 1e-6
    p.destroy()


# ---------------------------------------------------------------------------------------------
# Whole transforms vs the oracle NUFFT (1e-5 fp32, 1e-10 fp64) and vs the exact sums (10 eps)
# ---------------------------------------------------------------------------------------------

E2E_CASES = [
    WORKLOADS["2d_n64_m1e4_f32_e5"],                                   # full configuration
    Workload("e", 2, (100, 72), 50_001, 1e-5, "f32", seed=41),
    Workload("e", 2, (64, 64), 30_000, 1e-12, "f64", seed=42),
    Workload("e", 2, (33, 17), 5_000, 1e-9, "f64", seed=43),
    Workload("e", 3, (24, 20, 18), 40_000, 1e-5, "f32", seed=44),
    Workload("e", 3, (32, 32, 32), 40_000, 1e-2, "f32", seed=45),
    Workload("e", 3, (32, 32, 32), 60_000, 1e-5, "f32", dist="cluster", seed=46),
    Workload("e", 3, (20, 16, 12), 15_000, 1e-9, "f64", seed=47),
    Workload("e", 3, (16, 16, 16), 30_000, 1e-5, "f32", dist="box", seed=48),
    Workload("e", 3, (9, 16, 7), 2_000, 1e-12, "f64", seed=49),
    Workload("e", 1, (1024,), 100_000, 1e-5, "f32", seed=40),
    Workload("e", 1, (999,), 20_000, 1e-12, "f64", seed=401),
    Workload("e", 1, (5000,), 60_000, 1e-6, "f32", dist="cluster", seed=402),
    Workload("e", 1, (64,), 1_000, 1e-2, "f32", seed=403),
]


@pytest.mark.parametrize("wl", E2E_CASES, ids=lambda w: f"{w.dim}d_{w.N}_{w.M}_{w.precision}_{w.eps:g}_{w.dist}")
def test_type1_vs_oracle(nf, orc, wl):
    _announce(f"type1 {wl.N} M={wl.M} {wl.precision} eps={wl.eps} {wl.dist}")
    inp = make_inputs(wl, want_f=False)
    f = gpu_type1(nf, inp["X"], inp["c"], wl.N, wl.eps, wl.precision)
    ref = orc.nufft_type1(inp["X"], inp["c"], wl.N, wl.eps)
    err = orc.rel_l2(f, ref)
    assert err <= tol_for(wl.precision), err


@pytest.mark.parametrize("wl", E2E_CASES, ids=lambda w: f"{w.dim}d_{w.N}_{w.M}_{w.precision}_{w.eps:g}_{w.dist}")
def test_type2_vs_oracle(nf, orc, wl):
    _announce(f"type2 {wl.N} M={wl.M} {wl.precision} eps={wl.eps} {wl.dist}")
    inp = make_inputs(wl)
    c = gpu_type2(nf, inp["X"], inp["f"], wl.N, wl.eps, wl.precision)
    ref = orc.nufft_type2(inp["X"], inp["f"], wl.N, wl.eps)
    err = orc.rel_l2(c, ref)
    assert err <= tol_for(wl.precision), err


def test_small_config_vs_exact_sums(nf, orc):
    """2D 64x64 modes, M = 10,000, fp32 eps = 1e-5: both types within 10 eps of eqs. (1), (3)."""
    wl = WORKLOADS["2d_n64_m1e4_f32_e5"]
    inp = make_inputs(wl)
    f = gpu_type1(nf, inp["X"], inp["c"], wl.N, wl.eps, wl.precision)
    assert orc.rel_l2(f, orc.direct_type1(inp["X"], inp["c"], wl.N)) <= 10 * wl.eps
    c = gpu_type2(nf, inp["X"], inp["f"], wl.N, wl.eps, wl.precision)
    assert orc.rel_l2(c, orc.direct_type2(inp["X"], inp["f"], wl.N)) <= 10 * wl.eps


@pytest.mark.parametrize("N,prec,eps", [((64, 64), "f32", 1e-5), ((24, 20, 18), "f64", 1e-12),
                                         ((3000,), "f32", 1e-6), ((1001,), "f64", 1e-12)])
def test_adjointness_on_gpu(nf, N, prec, eps):
    """<type1(c), f> = <c, type2(f)> (the steps are exact transposes)."""
    wl = Workload("a", len(N), N, 20_000, eps, prec, seed=51)
    inp = make_inputs(wl)
    f1 = gpu_type1(nf, inp["X"], inp["c"], N, eps, prec).astype(np.complex128)
    c2 = gpu_type2(nf, inp["X"], inp["f"], N, eps, prec).astype(np.complex128)
    lhs = np.vdot(inp["f"].astype(np.complex128).ravel(), f1.ravel())
    rhs = np.vdot(c2, inp["c"].astype(np.complex128))
    rel = abs(lhs - rhs) / (np.linalg.norm(f1) * np.linalg.norm(inp["f"]))
    assert rel <= (1e-5 if prec == "f32" else 1e-12), rel


def test_methods_agree_and_caps(nf, orc):
    """GM, GM-sort and SM with several subproblem caps all match the oracle."""
    wl = Workload("m", 3, (24, 20, 18), 40_000, 1e-5, "f32", seed=52)
    inp = make_inputs(wl, want_f=False)
    ref = orc.nufft_type1(inp["X"], inp["c"], wl.N, wl.eps)
    for kw in ({"method": 1}, {"method": 3}, {"method": 2, "subproblem_cap": 1}, {"method": 2, "subproblem_cap": 100},
               {"method": 2, "bins": (8, 8, 8)}, {"method": 2, "bins": (4, 8, 16)}):
        f = gpu_type1(nf, inp["X"], inp["c"], wl.N, wl.eps, wl.precision, **kw)
        assert orc.rel_l2(f, ref) <= 1e-5, kw


def test_empty_and_single_point_1d(nf, orc):
    for prec in ("f32", "f64"):
        rd = np.float32 if prec == "f32" else np.float64
        cd = np.complex64 if prec == "f32" else np.complex128
        f = gpu_type1(nf, [np.zeros(0, rd)], np.zeros(0, cd), (40,), 1e-6, prec)
        assert np.all(f == 0)
        for x0 in (-math.pi, 0.3, np.nextafter(math.pi, 0)):
            X1 = [np.array([x0]).astype(rd)]
            f = gpu_type1(nf, X1, np.ones(1, cd), (41,), 1e-6, prec)
            ref = orc.nufft_type1(X1, np.ones(1, complex), (41,), 1e-6)
            assert orc.rel_l2(f, ref) <= tol_for(prec)


def test_empty_and_single_point(nf, orc):
    N = (16, 12)
    for prec in ("f32", "f64"):
        # M = 0: type 1 gives zeros, type 2 writes nothing
        X0 = [np.zeros(0, np.float32 if prec == "f32" else np.float64)] * 2
        f = gpu_type1(nf, X0, np.zeros(0, np.complex64), N, 1e-6, prec)
        assert np.all(f == 0)
        # M = 1: closed form exp(-i k.x0)
        x0 = [np.array([0.3], np.float64), np.array([-2.0], np.float64)]
        X1 = [x.astype(np.float32 if prec == "f32" else np.float64) for x in x0]
        f = gpu_type1(nf, X1, np.ones(1, np.complex64 if prec == "f32" else np.complex128), N, 1e-6, prec)
        ref = orc.nufft_type1(X1, np.ones(1, complex), N, 1e-6)
        assert orc.rel_l2(f, ref) <= tol_for(prec)


TINY_CASES = [((1,), "f32"), ((2,), "f64"), ((3,), "f32"), ((1, 1), "f64"), ((1, 5), "f32"), ((2, 3), "f64"),
              ((1, 1, 1), "f32"), ((3, 1, 2), "f64"), ((5, 4, 1), "f32"), ((2, 2, 2), "f64")]


@pytest.mark.parametrize("N,prec", TINY_CASES, ids=[f"{'x'.join(map(str, n))}_{p}" for n, p in TINY_CASES])
@pytest.mark.parametrize("M", [1, 3, 500])
def test_tiny_mode_counts(nf, orc, N, prec, M):
    """One to five modes per dimension: the fine grid is the kernel width or just above it, the
    padded bins wrap onto it several times, and a dimension with one mode has only k = 0; type 1
    and the adjoint type 2 match the oracle."""
    wl = Workload("tiny", len(N), N, M, 1e-6, prec, seed=161 + M)
    inp = make_inputs(wl)
    cd = cdtype(prec)
    p = nf.Plan(1, N, 1e-6, prec)
    p.setpts(*[to_dev(x) for x in inp["X"]])
    f = torch.empty(tuple(reversed(N)), dtype=cd, device=dev())
    c = torch.empty(M, dtype=cd, device=dev())
    p.execute(to_dev(inp["c"]), f)
    p.execute_adjoint(c, to_dev(inp["f"]))
    torch.cuda.synchronize()
    assert p.range_errors() == 0
    p.destroy()
    e1 = orc.rel_l2(f.cpu().numpy(), orc.nufft_type1(inp["X"], inp["c"], N, 1e-6))
    e2 = orc.rel_l2(c.cpu().numpy(), orc.nufft_type2(inp["X"], inp["f"], N, 1e-6))
    assert e1 <= tol_for(prec) and e2 <= tol_for(prec), (e1, e2)


SIGMA_CASES = [
    Workload("sg", 1, (2000,), 40_000, 1e-6, "f32", seed=111),
    Workload("sg", 2, (100, 72), 50_001, 1e-5, "f32", seed=112),
    Workload("sg", 2, (64, 48), 20_000, 1e-12, "f64", seed=113),
    Workload("sg", 3, (24, 20, 18), 40_000, 1e-5, "f32", seed=114),
    Workload("sg", 3, (20, 16, 12), 15_000, 1e-9, "f64", seed=115),
    Workload("sg", 3, (32, 32, 32), 60_000, 1e-5, "f32", dist="cluster", seed=116),
]


def _sigma_tol(prm, prec, M=None):
    """Parity bar for sigma < 2, derived from the arithmetic.  The fine grid is rounded to the
    plan precision (unit roundoff u) and the FFT adds O(log n) roundings of that size; the
    correction of eq. (10) scales mode k by p(k), so the output's relative error is about
    u kappa with kappa = rms(p / p_min) rms(p_min / p).  For type 1 (M given) each cell also
    sums K = M w^d / n^d contributions (on average), partly in the plan precision (the 3D
    column runs accumulate in registers before the fp64 LDS bin) and in another order than the
    oracle's: another u sqrt(K) kappa.  At sigma = 2 kappa is a few units; at sigma = 1.25 in
    3D it reaches hundreds (fp32, w = 9) to millions (fp64, w = 15).  Bar: max(1e-5 fp32 /
    1e-10 fp64, 4 kappa u (1 + sqrt(1 + K))) for type 1, max(.., 4 kappa u) for type 2."""
    P = np.abs(orc_outer(prm))
    pm = P.min()
    kappa = math.sqrt(np.mean((P / pm) ** 2)) * math.sqrt(np.mean((pm / P) ** 2))
    u = 2.0 ** -24 if prec == "f32" else 2.0 ** -53
    acc = 0.0
    if M is not None:
        K = M * prm.w ** prm.dim / float(np.prod(prm.n))
        acc = u * math.sqrt(1.0 + K)
    return max(tol_for(prec), 4 * kappa * (u + acc))


def orc_outer(prm):
    out = np.array(1.0)
    for p in prm.p[::-1]:
        out = np.multiply.outer(out, p)
    return out


@pytest.mark.parametrize("wl", SIGMA_CASES, ids=lambda w: f"{w.dim}d_{w.N}_{w.precision}_{w.eps:g}_{w.dist}")
@pytest.mark.parametrize("sigma", [1.25, 1.5])
def test_upsampfac_vs_oracle(nf, orc, wl, sigma):
    """sigma < 2: the plan's w, beta and fine grid equal the oracle's, and both types match the
    oracle NUFFT at the same sigma, within the bar derived in _sigma_tol."""
    _announce(f"sigma={sigma} {wl.N} M={wl.M} {wl.precision} eps={wl.eps} {wl.dist}")
    inp = make_inputs(wl)
    prm = orc.Params(wl.N, wl.eps, sigma)
    p = nf.Plan(1, wl.N, wl.eps, wl.precision, upsampfac=sigma)
    info = p.info()
    assert info["w"] == prm.w and info["n"] == prm.n and info["sigma"] == sigma
    assert abs(info["beta"] - prm.beta) <= 1e-12 * prm.beta
    p.setpts(*[to_dev(x) for x in inp["X"]])
    cd = cdtype(wl.precision)
    f = torch.empty(tuple(reversed(wl.N)), dtype=cd, device=dev())
    c = torch.empty(wl.M, dtype=cd, device=dev())
    p.execute(to_dev(inp["c"]), f)
    p.execute_adjoint(c, to_dev(inp["f"]))
    torch.cuda.synchronize()
    p.destroy()
    e1 = orc.rel_l2(f.cpu().numpy(), orc.nufft_type1(inp["X"], inp["c"], wl.N, wl.eps, sigma))
    e2 = orc.rel_l2(c.cpu().numpy(), orc.nufft_type2(inp["X"], inp["f"], wl.N, wl.eps, sigma))
    tol1, tol2 = _sigma_tol(prm, wl.precision, wl.M), _sigma_tol(prm, wl.precision)
    assert e1 <= tol1 and e2 <= tol2, (e1, e2, tol1, tol2)


def test_type2_bitwise_reproducible_type1_close(nf):
    wl = Workload("r", 3, (32, 32, 32), 50_000, 1e-5, "f32", seed=53)
    inp = make_inputs(wl)
    a = gpu_type2(nf, inp["X"], inp["f"], wl.N, wl.eps, wl.precision)
    b = gpu_type2(nf, inp["X"], inp["f"], wl.N, wl.eps, wl.precision)
    np.testing.assert_array_equal(a, b)
    f1 = gpu_type1(nf, inp["X"], inp["c"], wl.N, wl.eps, wl.precision)
    f2 = gpu_type1(nf, inp["X"], inp["c"], wl.N, wl.eps, wl.precision)
    assert np.linalg.norm(f1 - f2) <= 1e-6 * np.linalg.norm(f1)


def test_repeated_execute_and_resetpts(nf, orc):
    """One plan: several executes with new strengths, then new points (plan reuse)."""
    N = (40, 36)
    p = nf.Plan(1, N, 1e-5, "f32")
    f = torch.empty((36, 40), dtype=torch.complex64, device=dev())
    for seed in (61, 62):
        wl = Workload("p", 2, N, 7_000 + seed, 1e-5, "f32", seed=seed)
        inp = make_inputs(wl, want_f=False)
        p.setpts(*[to_dev(x) for x in inp["X"]])
        for k in range(2):
            c = inp["c"] * (k + 1)
            p.execute(to_dev(c), f)
            torch.cuda.synchronize()
            ref = orc.nufft_type1(inp["X"], c, N, 1e-5)
            assert orc.rel_l2(f.cpu().numpy(), ref) <= 1e-5
    p.destroy()


def test_stage_times_average_and_reset(nf):
    """Stage times average the calls since the previous read (the last 16 when there are
    more); a stage not run since then keeps its value, a direction never run reads zero."""
    import torch
    wl = Workload("tm", 2, (64, 48), 20_000, 1e-5, "f32", seed=141)
    inp = make_inputs(wl, want_f=False)
    p = nf.Plan(1, wl.N, wl.eps, wl.precision, timing=True)
    c = to_dev(inp["c"])
    f = torch.empty(tuple(reversed(wl.N)), dtype=cdtype(wl.precision), device=dev())
    p.setpts(*[to_dev(x) for x in inp["X"]])
    p.execute(c, f)
    st1 = p.stage_times()
    assert st1["sort"] > 0 and st1["spread"] > 0 and st1["fft1"] > 0
    assert st1["interp"] == 0 and st1["fft2"] == 0
    for _ in range(20):   # more executes than the event ring holds
        p.execute(c, f)
    st2 = p.stage_times()
    assert st2["sort"] == st1["sort"]
    assert st2["spread"] > 0 and st2["deconv"] > 0
    p.destroy()


@pytest.mark.parametrize("wl", [Workload("adj", 3, (24, 20, 18), 40_000, 1e-5, "f32", seed=71),
                                Workload("adj", 2, (64, 48), 20_000, 1e-12, "f64", seed=72)],
                         ids=["3d_f32", "2d_f64"])
def test_execute_adjoint_matches_oracle(nf, orc, wl):
    """A type 1 plan runs type 2 on its sorted points and vice versa (one sort for the pair)."""
    inp = make_inputs(wl)
    X = [to_dev(x) for x in inp["X"]]
    cd = cdtype(wl.precision)
    ref1 = orc.nufft_type1(inp["X"], inp["c"], wl.N, wl.eps)
    ref2 = orc.nufft_type2(inp["X"], inp["f"], wl.N, wl.eps)
    for t in (1, 2):
        p = nf.Plan(t, wl.N, wl.eps, wl.precision, timing=True)
        p.setpts(*X)
        f = torch.empty(tuple(reversed(wl.N)), dtype=cd, device=dev())
        c = torch.empty(wl.M, dtype=cd, device=dev())
        if t == 1:
            p.execute(to_dev(inp["c"]), f)
            p.execute_adjoint(c, to_dev(inp["f"]))
        else:
            p.execute(c, to_dev(inp["f"]))
            p.execute_adjoint(to_dev(inp["c"]), f)
        torch.cuda.synchronize()
        assert orc.rel_l2(f.cpu().numpy(), ref1) <= tol_for(wl.precision)
        assert orc.rel_l2(c.cpu().numpy(), ref2) <= tol_for(wl.precision)
        st = p.stage_times()
        assert st["sort"] > 0 and st["spread"] > 0 and st["interp"] > 0 and st["fft1"] > 0 and st["fft2"] > 0
        p.destroy()


# ---------------------------------------------------------------------------------------------
# The point-patch spreader (2D, and 3D outside the column widths) across kernel widths
# ---------------------------------------------------------------------------------------------

PATCH_CASES = [(2, "f32", 1e-1), (2, "f32", 1e-3), (2, "f32", 1e-6), (2, "f64", 1e-8), (2, "f64", 1e-10),
               (2, "f64", 1e-13), (2, "f64", 1e-15), (3, "f32", 1e-1), (3, "f32", 1e-3), (3, "f64", 1e-2),
               (3, "f64", 1e-3), (3, "f64", 1e-12), (3, "f64", 1e-13), (3, "f64", 1e-15)]


@pytest.mark.parametrize("dim,prec,eps", PATCH_CASES, ids=[f"{d}d_{p}_{e:g}" for d, p, e in PATCH_CASES])
def test_point_patch_widths(nf, orc, dim, prec, eps):
    """Plans served by the point-patch spreader at kernel widths 2..16 (the staged point record's
    padded rows change with w): the plan reports no column order, and type 1 plus the adjoint type 2
    on the same sorted points match the oracle."""
    N = (40, 36) if dim == 2 else (16, 14, 12)
    wl = Workload("patch", dim, N, 8_000 if dim == 2 else 6_000, eps, prec, seed=141)
    _announce(f"point-patch widths {dim}D {prec} eps={eps}")
    inp = make_inputs(wl)
    cd = cdtype(prec)
    p = nf.Plan(1, N, eps, prec)
    info = p.info()
    assert info["colw"] == 0, info
    p.setpts(*[to_dev(x) for x in inp["X"]])
    f = torch.empty(tuple(reversed(N)), dtype=cd, device=dev())
    c = torch.empty(wl.M, dtype=cd, device=dev())
    p.execute(to_dev(inp["c"]), f)
    p.execute_adjoint(c, to_dev(inp["f"]))
    torch.cuda.synchronize()
    assert p.range_errors() == 0
    p.destroy()
    e1 = orc.rel_l2(f.cpu().numpy(), orc.nufft_type1(inp["X"], inp["c"], N, eps))
    e2 = orc.rel_l2(c.cpu().numpy(), orc.nufft_type2(inp["X"], inp["f"], N, eps))
    assert e1 <= tol_for(prec) and e2 <= tol_for(prec), (info["w"], e1, e2)


WIDTH_METHOD_CASES = [(1, "f32", 1e-1, 2), (1, "f32", 1e-3, 2), (1, "f64", 1e-8, 2), (1, "f64", 1e-13, 2),
                      (1, "f64", 1e-15, 2), (1, "f64", 1e-13, 1), (2, "f32", 1e-1, 1), (2, "f64", 1e-13, 1),
                      (3, "f64", 1e-15, 1), (1, "f32", 1e-1, 3), (2, "f64", 1e-15, 3), (3, "f64", 1e-13, 3)]


@pytest.mark.parametrize("dim,prec,eps,method", WIDTH_METHOD_CASES,
                         ids=[f"{d}d_{p}_{e:g}_m{m}" for d, p, e, m in WIDTH_METHOD_CASES])
def test_widths_1d_and_gm(nf, orc, dim, prec, eps, method):
    """The kernels outside the 2D/3D point-patch and column spreaders at the extreme kernel widths:
    the 1D SM spreader and interpolation (w = 2, 4, 9, 14, 16) and the GM-sort (method 1) and GM
    (method 3) kernels in 1D, 2D and 3D (w = 2, 14, 16); type 1 and the adjoint type 2 match the
    oracle."""
    N = {1: (300,), 2: (40, 36), 3: (16, 14, 12)}[dim]
    wl = Workload("wm", dim, N, 5_000, eps, prec, seed=151)
    _announce(f"widths {dim}D {prec} eps={eps} method={method}")
    inp = make_inputs(wl)
    cd = cdtype(prec)
    p = nf.Plan(1, N, eps, prec, method=method)
    p.setpts(*[to_dev(x) for x in inp["X"]])
    f = torch.empty(tuple(reversed(N)), dtype=cd, device=dev())
    c = torch.empty(wl.M, dtype=cd, device=dev())
    p.execute(to_dev(inp["c"]), f)
    p.execute_adjoint(c, to_dev(inp["f"]))
    torch.cuda.synchronize()
    assert p.range_errors() == 0
    p.destroy()
    e1 = orc.rel_l2(f.cpu().numpy(), orc.nufft_type1(inp["X"], inp["c"], N, eps))
    e2 = orc.rel_l2(c.cpu().numpy(), orc.nufft_type2(inp["X"], inp["f"], N, eps))
    assert e1 <= tol_for(prec) and e2 <= tol_for(prec), (e1, e2)


# ---------------------------------------------------------------------------------------------
# The 3D column-run spreader at every kernel width it serves
# ---------------------------------------------------------------------------------------------

# fp32 up to w = 8 runs two 768-lane workgroups per CU, above that one 1024-lane workgroup
COLUMN_CASES = [("f32", 1e-4), ("f32", 1e-6), ("f32", 1e-7), ("f32", 1e-8), ("f32", 1e-10)] + \
               [("f64", e) for e in (1e-4, 1e-5, 1e-6, 1e-7, 1e-8, 1e-10, 1e-11)]


@pytest.mark.parametrize("prec,eps", COLUMN_CASES, ids=[f"{p}_{e:g}" for p, e in COLUMN_CASES])
def test_column_kernel_widths(nf, orc, prec, eps):
    """3D plans whose kernel width selects the column-run spreader (w = 5..12): the plan reports the
    column order, and type 1 plus the adjoint type 2 on the same sorted points match the oracle."""
    N = (20, 18, 16)
    wl = Workload("col", 3, N, 12_000, eps, prec, seed=81)
    _announce(f"column widths {prec} eps={eps}")
    inp = make_inputs(wl)
    cd = cdtype(prec)
    p = nf.Plan(1, N, eps, prec)
    info = p.info()
    assert info["colw"] == info["w"] and info["colstep"] >= 1, info
    p.setpts(*[to_dev(x) for x in inp["X"]])
    f = torch.empty(tuple(reversed(N)), dtype=cd, device=dev())
    c = torch.empty(wl.M, dtype=cd, device=dev())
    p.execute(to_dev(inp["c"]), f)
    p.execute_adjoint(c, to_dev(inp["f"]))
    torch.cuda.synchronize()
    p.destroy()
    e1 = orc.rel_l2(f.cpu().numpy(), orc.nufft_type1(inp["X"], inp["c"], N, eps))
    e2 = orc.rel_l2(c.cpu().numpy(), orc.nufft_type2(inp["X"], inp["f"], N, eps))
    assert e1 <= tol_for(prec) and e2 <= tol_for(prec), (info["w"], e1, e2)


@pytest.mark.parametrize("bins,dist", [(None, "box"), (None, "uniform"), ((32, 16, 8), "uniform"),
                                       ((16, 8, 8), "box")],
                         ids=["default_box", "default_uniform", "32x16x8_uniform", "16x8x8_box"])
def test_column_fp32_bins(nf, orc, bins, dist):
    """fp32 column-run plans (w = 6) keep the padded bin in fp32 and add each register z-line into
    it by compare-and-swap, retrying a cell whose swap lost to another wavefront's overlapping
    column block.  Every point in one 8-cell box with the full subproblem cap puts all wavefronts
    of a workgroup on the same columns (the most retries); 32 x 16 x 8 bins fit the LDS once (one
    workgroup per CU), the default 16 x 16 x 8 twice.  The spread step matches the oracle's spread
    at the single-step bar, and type 1 plus the adjoint type 2 match the oracle NUFFT."""
    N = (24, 20, 16)
    wl = Workload("cc", 3, N, 40_000, 1e-5, "f32", dist=dist, seed=171)
    _announce(f"column fp32 bins={bins} {dist}")
    inp = make_inputs(wl)
    kw = {"bins": bins} if bins else {}
    p = nf.Plan(1, N, wl.eps, "f32", **kw)
    info = p.info()
    assert info["w"] == 6 and info["colw"] == 6, info
    assert tuple(info["bins"]) == (bins or (16, 16, 8)), info
    X = [to_dev(x) for x in inp["X"]]
    p.setpts(*X)
    grid = torch.empty(p.fine_cells, dtype=torch.complex64, device=dev())
    p.spread(to_dev(inp["c"]), grid)
    f = torch.empty(tuple(reversed(N)), dtype=torch.complex64, device=dev())
    c = torch.empty(wl.M, dtype=torch.complex64, device=dev())
    p.execute(to_dev(inp["c"]), f)
    p.execute_adjoint(c, to_dev(inp["f"]))
    torch.cuda.synchronize()
    ref = orc.spread(inp["X"], inp["c"], p.n, p.w, p.beta)
    assert orc.rel_l2(grid.cpu().numpy(), ref.ravel()) <= _step_tol("f32")
    assert orc.rel_l2(f.cpu().numpy(), orc.nufft_type1(inp["X"], inp["c"], N, wl.eps)) <= tol_for("f32")
    assert orc.rel_l2(c.cpu().numpy(), orc.nufft_type2(inp["X"], inp["f"], N, wl.eps)) <= tol_for("f32")
    assert p.range_errors() == 0
    p.destroy()


@pytest.mark.parametrize("wl", [Workload("gm", 3, (24, 20, 18), 30_000, 1e-5, "f32", seed=91),
                                Workload("gm", 2, (48, 40), 20_000, 1e-12, "f64", seed=92),
                                Workload("gm", 3, (20, 16, 12), 10_000, 1e-9, "f64", dist="cluster", seed=93),
                                Workload("gm", 1, (3000,), 50_000, 1e-6, "f32", seed=94)],
                         ids=["3d_f32", "2d_f64", "3d_f64_cluster", "1d_f32"])
def test_gm_method(nf, orc, wl):
    """GM (Sec. III-A): setpts keeps the caller's order (identity permutation, no subproblems, no
    binning: the bin counts read zero); type 1 and the adjoint type 2 match the oracle NUFFT."""
    _announce(f"GM {wl.N} {wl.precision} eps={wl.eps} {wl.dist}")
    inp = make_inputs(wl)
    X = [to_dev(x) for x in inp["X"]]
    p = nf.Plan(1, wl.N, wl.eps, wl.precision, method=3)
    p.setpts(*X)
    info = p.info()
    assert info["method"] == 3 and info["nsubproblems"] == 0 and info["colw"] == 0
    perm, counts, sub = p.get_sort()
    assert sub.numel() == 0
    np.testing.assert_array_equal(perm.cpu().numpy(), np.arange(wl.M))
    assert not counts.cpu().numpy().any()
    cd = cdtype(wl.precision)
    f = torch.empty(tuple(reversed(wl.N)), dtype=cd, device=dev())
    c = torch.empty(wl.M, dtype=cd, device=dev())
    p.execute(to_dev(inp["c"]), f)
    p.execute_adjoint(c, to_dev(inp["f"]))
    torch.cuda.synchronize()
    p.destroy()
    # GM adds every contribution with a global atomic in the plan precision (fp32: 1e-5, as for
    # GM-sort spreading)
    assert orc.rel_l2(f.cpu().numpy(), orc.nufft_type1(inp["X"], inp["c"], wl.N, wl.eps)) <= tol_for(wl.precision)
    assert orc.rel_l2(c.cpu().numpy(), orc.nufft_type2(inp["X"], inp["f"], wl.N, wl.eps)) <= tol_for(wl.precision)
