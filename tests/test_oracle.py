"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: each check uses a closed form, a
library routine computing the same quantity another way, a brute-force sum over
the whole grid, a printed table, or an identity the exact transforms satisfy.
"""
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.special

from nonuniform_fft_amd.workloads import WORKLOADS, Workload, make_inputs, scaled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_complex(rng, shape):
    return rng.standard_normal(shape) + 1j * rng.standard_normal(shape)


def _uniform_points(rng, d, M):
    return [rng.uniform(-math.pi, math.pi, M) for _ in range(d)]


# ---------------------------------------------------------------------------------------------
# Plan parameters
# ---------------------------------------------------------------------------------------------

def test_width_table_printed_on_pages(oracle_mod):
    """Width rule of eq. (6) against the tolerance->width values the pages print."""
    rows = []
    with open(os.path.join(GOLDEN, "es_width.txt")) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                e, w = line.split()
                rows.append((float(e), int(w)))
    assert len(rows) == 5
    for eps, w in rows:
        assert oracle_mod.kernel_params(eps)[0] == w, eps


def test_width_between_table_entries(oracle_mod):
    # log10(1/eps) not an integer: w = ceil(.) + 1
    assert oracle_mod.kernel_params(2e-6)[0] == 7
    assert oracle_mod.kernel_params(0.5e-2)[0] == 4
    assert oracle_mod.kernel_params(1e-2)[0] == 3
    # clamps
    assert oracle_mod.kernel_params(1e-30)[0] == 16
    assert oracle_mod.kernel_params(0.9)[0] == 2


def test_fine_size_against_enumeration(oracle_mod):
    """Smallest 2^a 3^b 5^c >= max(2N, w): compare with a sorted enumeration of 5-smooth numbers."""
    smooth = sorted({2 ** a * 3 ** b * 5 ** c for a in range(14) for b in range(9) for c in range(7)})
    for N in list(range(1, 300)) + [500, 513, 1000, 1024, 1025, 2047]:
        for w in (2, 6, 13, 16):
            target = max(2 * N, w)
            expect = next(s for s in smooth if s >= target)
            assert oracle_mod.fine_size(N, w) == expect, (N, w)


def test_fine_size_sigma_below_two(oracle_mod):
    """sigma < 2: smallest 5-smooth number >= max(ceil(sigma N), w), against an enumeration."""
    smooth = sorted({2 ** a * 3 ** b * 5 ** c for a in range(14) for b in range(9) for c in range(7)})
    for sigma in (1.25, 1.5):
        for N in list(range(1, 200)) + [1000, 1023]:
            for w in (4, 9):
                target = max(-(-int(sigma * 4) * N // 4), w)      # ceil(sigma N) in integers
                expect = next(s for s in smooth if s >= target)
                assert oracle_mod.fine_size(N, w, sigma) == expect, (sigma, N, w)
    with pytest.raises(ValueError):
        oracle_mod.kernel_params(1e-6, 1.1)
    with pytest.raises(ValueError):
        oracle_mod.kernel_params(1e-6, 2.5)


# ---------------------------------------------------------------------------------------------
# Kernel and its Fourier transform (eqs. (4), (5))
# ---------------------------------------------------------------------------------------------

def test_es_kernel_values(oracle_mod):
    beta = 13.8
    assert oracle_mod.es_kernel(0.0, beta) == 1.0
    assert oracle_mod.es_kernel(1.0, beta) == pytest.approx(math.exp(-beta), rel=1e-15)
    assert oracle_mod.es_kernel(-1.0, beta) == pytest.approx(math.exp(-beta), rel=1e-15)
    assert oracle_mod.es_kernel(1.0 + 1e-12, beta) == 0.0
    assert oracle_mod.es_kernel(0.6, beta) == pytest.approx(math.exp(beta * (0.8 - 1.0)), rel=1e-15)


def test_phihat_beta_zero_is_sinc(oracle_mod):
    """beta = 0 turns the kernel into the indicator of [-1, 1]: transform 2 sin(xi)/xi."""
    xi = np.linspace(0.01, 20.0, 57)
    got = oracle_mod.phihat(xi, 1, 0.0)
    np.testing.assert_allclose(got, 2 * np.sin(xi) / xi, rtol=1e-13, atol=1e-14)


def test_phihat_at_zero_struve_closed_form(oracle_mod):
    """int_{-1}^{1} exp(beta sqrt(1-z^2)) dz = pi (I_1(beta) + L_{-1}(beta)) (modified Bessel and
    modified Struve functions; z = sin(theta) splits the integrand into cosh and sinh parts)."""
    for w in range(2, 17):
        beta = 2.30 * w
        expect = math.exp(-beta) * math.pi * (scipy.special.iv(1, beta) + scipy.special.modstruve(-1, beta))
        assert oracle_mod.phihat(np.array([0.0]), w, beta)[0] == pytest.approx(expect, rel=1e-12)


@pytest.mark.parametrize("w", [2, 3, 6, 10, 13, 16])
def test_phihat_adaptive_quadrature(oracle_mod, w):
    """The transform by scipy's adaptive quadrature of eq. (4) directly in z."""
    beta = 2.30 * w
    for xi in (0.0, 0.7, w * math.pi / 4, w * math.pi / 2 * 0.97):
        f = lambda z: math.exp(beta * (math.sqrt(max(0.0, 1 - z * z)) - 1)) * math.cos(xi * z)
        ref, _ = scipy.integrate.quad(f, -1, 1, epsabs=1e-15, epsrel=1e-14, limit=400)
        got = oracle_mod.phihat(np.array([xi]), w, beta)[0]
        assert got == pytest.approx(ref, rel=1e-11, abs=1e-15)


# ---------------------------------------------------------------------------------------------
# Exact sums (eqs. (1), (3))
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("N", [(16,), (9,), (8, 6), (5, 7), (4, 6, 5)])
def test_direct_type1_on_uniform_grid_is_fft(oracle_mod, N):
    """Points on the equispaced grid 2 pi j / N - pi: eq. (1) is (-1)^(sum k) times numpy's FFT."""
    rng = _rng(1)
    d = len(N)
    axes = [2 * np.pi * np.arange(Ni) / Ni - np.pi for Ni in N]
    mesh = np.meshgrid(*axes[::-1], indexing="ij")[::-1]       # arrays shaped (N3, N2, N1)
    X = [m.ravel() for m in mesh]
    c = _rand_complex(rng, tuple(reversed(N)))
    got = oracle_mod.direct_type1(X, c.ravel(), N)
    F = np.fft.fftn(c)
    ks = [oracle_mod.mode_range(Ni) for Ni in N][::-1]
    K = np.meshgrid(*ks, indexing="ij")
    expect = F[np.ix_(*[k % Ni for k, Ni in zip(ks, tuple(reversed(N)))])]
    expect = expect * np.where(sum(K) % 2 == 0, 1.0, -1.0)
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-12 * np.abs(expect).max())


@pytest.mark.parametrize("N", [(11,), (6, 9), (4, 5, 3)])
def test_direct_type2_all_ones_is_dirichlet_product(oracle_mod, N):
    """f = 1 on I_N: c_j = prod_i sum_{k in I_Ni} exp(i k x_ij) (geometric series)."""
    rng = _rng(2)
    X = _uniform_points(rng, len(N), 40)
    got = oracle_mod.direct_type2(X, np.ones(int(np.prod(N)), complex), N)
    expect = np.ones(40, complex)
    for x, Ni in zip(X, N):
        a = -(Ni // 2)
        e = np.exp(1j * x)
        expect *= np.exp(1j * a * x) * (1 - e ** Ni) / (1 - e)
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("N", [(13,), (7, 8), (4, 6, 5)])
def test_direct_sums_are_adjoint(oracle_mod, N):
    rng = _rng(3)
    M = 37
    X = _uniform_points(rng, len(N), M)
    c = _rand_complex(rng, M)
    f = _rand_complex(rng, tuple(reversed(N)))
    lhs = np.vdot(f.ravel(), oracle_mod.direct_type1(X, c, N).ravel())
    rhs = np.vdot(oracle_mod.direct_type2(X, f, N), c)
    assert abs(lhs - rhs) <= 1e-12 * abs(lhs)


def test_direct_selected_entries_match_full(oracle_mod):
    rng = _rng(4)
    N = (6, 5, 4)
    X = _uniform_points(rng, 3, 30)
    c = _rand_complex(rng, 30)
    full = oracle_mod.direct_type1(X, c, N).ravel()
    sel = np.array([0, 7, 33, 119])
    np.testing.assert_array_equal(oracle_mod.direct_type1(X, c, N, sel=sel), full[sel])
    f = _rand_complex(rng, (4, 5, 6))
    full2 = oracle_mod.direct_type2(X, f, N)
    np.testing.assert_array_equal(oracle_mod.direct_type2(X, f, N, sel=[3, 29, 0]), full2[[3, 29, 0]])


@pytest.mark.parametrize("N", [(7,), (6, 5), (5, 4, 6)])
def test_direct_type2_modes_matches_dense(oracle_mod, N):
    """The sparse form of eq. (3) equals the dense exact sum of the C oracle on an f that is zero
    except at the listed modes (odd and even N, corner modes included)."""
    rng = _rng(5)
    d = len(N)
    X = _uniform_points(rng, d, 25)
    total = int(np.prod(N))
    modes = np.array(sorted({0, total - 1, *rng.integers(0, total, 6).tolist()}), dtype=np.int64)
    vals = _rand_complex(rng, modes.size)
    f = np.zeros(total, dtype=complex)
    f[modes] = vals
    dense = oracle_mod.direct_type2(X, f.reshape(tuple(reversed(N))), N)
    sparse = oracle_mod.direct_type2_modes(X, N, modes, vals)
    assert np.max(np.abs(sparse - dense)) <= 1e-13 * np.max(np.abs(dense))


# ---------------------------------------------------------------------------------------------
# Spreading / interpolation against a brute-force periodic sum over the whole grid (eqs. (7), (8))
# ---------------------------------------------------------------------------------------------

def _brute_psi_per(X, n, w, beta):
    """Matrix Psi[l, j] = psi_per(l h - pi - x_j) over every fine cell l (first index fastest),
    summing periodic images directly from eq. (8); no stencil logic.  The support is taken
    half-open, -1 <= z < 1: when a point sits exactly w/2 cells from a cell on both sides
    (a tie), the method keeps w cells, dropping the far endpoint (value exp(-beta))."""
    d = len(n)
    alpha = [w * math.pi / ni for ni in n]
    M = len(X[0])
    per_dim = []
    for i in range(d):
        l = np.arange(n[i])[:, None]
        acc = np.zeros((n[i], M))
        for m in range(-3, 4):
            u = l * (2 * math.pi / n[i]) - math.pi - X[i][None, :] - 2 * math.pi * m
            z = u / alpha[i]
            inside = (z >= -1) & (z < 1)
            acc += np.where(inside, np.exp(beta * (np.sqrt(np.clip(1 - z * z, 0, None)) - 1)), 0.0)
        per_dim.append(acc)
    # tensor product: cell index l1 + n1 (l2 + n2 l3)
    out = per_dim[0]
    for i in range(1, d):
        out = (per_dim[i][:, None, :] * out[None, :, :]).reshape(-1, M)
    return out


@pytest.mark.parametrize("n,w", [((40,), 6), ((30,), 13), ((16, 12), 6), ((12, 10), 3), ((10, 8, 12), 4),
                                 ((9, 8, 10), 5)])
def test_spread_and_interp_match_bruteforce(oracle_mod, n, w):
    rng = _rng(5)
    beta = 2.30 * w
    M = 23
    X = _uniform_points(rng, len(n), M)
    # include points at the ends of the periodic box, and points in the folded ranges
    # [pi, 3 pi) and [-3 pi, -pi), which the method maps back by one period (values off the grid
    # points: where t - w/2 is an integer the support is a tie of two equal endpoint weights,
    # and which end a rounding picks is not fixed by eq. (8))
    X[0][0] = -math.pi
    X[0][1] = math.pi - 1e-13
    X[0][2] = math.pi + 1e-3
    X[0][3] = 2.5 * math.pi + 0.01
    X[0][4] = -2.2 * math.pi
    X[0][5] = np.nextafter(-math.pi, -4.0)
    X[-1][6] = 3 * math.pi - 1e-9
    X[-1][7] = -3 * math.pi + 0.013
    c = _rand_complex(rng, M)
    P = _brute_psi_per(X, n, w, beta)
    b = oracle_mod.spread(X, c, n, w, beta)
    ref = P @ c
    np.testing.assert_allclose(b.ravel(), ref, rtol=1e-12, atol=1e-11 * np.abs(ref).max())
    g = _rand_complex(rng, tuple(reversed(n)))
    cc = oracle_mod.interp(X, g, w, beta)
    ref2 = P.T @ g.ravel()
    np.testing.assert_allclose(cc, ref2, rtol=1e-12, atol=1e-11 * np.abs(ref2).max())


# ---------------------------------------------------------------------------------------------
# Whole NUFFT against the exact sums (accuracy statement after eq. (6))
# ---------------------------------------------------------------------------------------------

CASES = [
    ((256,), 5000, 1e-5, "f32"),           # 1D
    ((100,), 1000, 1e-12, "f64"),
    ((63,), 300, 1e-2, "f32"),
    ((64, 64), 10_000, 1e-5, "f32"),       # the 2D 64x64 configuration at full size
    ((32, 32), 1000, 1e-2, "f32"),
    ((32, 32), 1000, 1e-9, "f64"),
    ((32, 32), 1000, 1e-12, "f64"),
    ((16, 16, 16), 4096, 1e-5, "f32"),      # 3D validation size used by the HP-NFFT page
    ((16, 16, 16), 4096, 1e-2, "f32"),
    ((16, 16, 16), 4096, 1e-9, "f64"),
    ((12, 10, 9), 777, 1e-12, "f64"),       # odd sizes
    ((33, 17), 501, 1e-6, "f64"),
]


@pytest.mark.parametrize("N,M,eps,prec", CASES)
def test_nufft_vs_direct_within_10eps(oracle_mod, N, M, eps, prec):
    wl = Workload(name="t", dim=len(N), N=N, M=M, eps=eps, precision=prec, seed=11)
    inp = make_inputs(wl)
    X, c, f = inp["X"], inp["c"], inp["f"]
    f1 = oracle_mod.nufft_type1(X, c, N, eps)
    fd = oracle_mod.direct_type1(X, c, N)
    assert oracle_mod.rel_l2(f1, fd) <= 10 * eps
    c2 = oracle_mod.nufft_type2(X, f, N, eps)
    cd = oracle_mod.direct_type2(X, f, N)
    assert oracle_mod.rel_l2(c2, cd) <= 10 * eps


SIGMA_CASES = [
    ((300,), 2000, 1e-3, 1.25), ((300,), 2000, 1e-9, 1.25), ((257,), 1500, 1e-6, 1.5),
    ((32, 28), 1500, 1e-4, 1.25), ((32, 32), 1000, 1e-12, 1.5), ((24, 20), 1200, 1e-6, 1.5),
    ((12, 10, 9), 900, 1e-3, 1.25), ((12, 12, 12), 900, 1e-6, 1.25), ((10, 9, 8), 700, 1e-9, 1.5),
]


@pytest.mark.parametrize("N,M,eps,sigma", SIGMA_CASES)
def test_nufft_sigma_below_two_vs_direct(oracle_mod, N, M, eps, sigma):
    """Upsampling sigma < 2 with the width and shape of the reading: both types within 10 eps of
    the exact sums (eqs. (1), (3)), the accuracy statement after eq. (6)."""
    wl = Workload(name="t", dim=len(N), N=N, M=M, eps=eps, precision="f64", seed=13)
    inp = make_inputs(wl)
    X, c, f = inp["X"], inp["c"], inp["f"]
    prm = oracle_mod.Params(N, eps, sigma)
    assert all(ni < 2 * Ni or ni == prm.w or ni <= 8 for ni, Ni in zip(prm.n, N))
    assert oracle_mod.rel_l2(oracle_mod.nufft_type1(X, c, N, eps, sigma), oracle_mod.direct_type1(X, c, N)) <= 10 * eps
    assert oracle_mod.rel_l2(oracle_mod.nufft_type2(X, f, N, eps, sigma), oracle_mod.direct_type2(X, f, N)) <= 10 * eps


def test_nufft_sigma_adjoint(oracle_mod):
    rng = _rng(14)
    N, eps, sigma = (40, 30), 1e-7, 1.25
    X = _uniform_points(rng, 2, 250)
    c = _rand_complex(rng, 250)
    f = _rand_complex(rng, (30, 40))
    lhs = np.vdot(f.ravel(), oracle_mod.nufft_type1(X, c, N, eps, sigma).ravel())
    rhs = np.vdot(oracle_mod.nufft_type2(X, f, N, eps, sigma), c)
    assert abs(lhs - rhs) <= 1e-13 * abs(lhs)


# ---------------------------------------------------------------------------------------------
# Type 3 (nonuniform to nonuniform)
# ---------------------------------------------------------------------------------------------

def test_direct_type3_on_integer_targets_is_type1(oracle_mod):
    """Targets s = -k on the modes I_N: the type 3 sum is the type 1 sum of eq. (1)."""
    rng = _rng(21)
    N = (6, 5, 4)
    X = _uniform_points(rng, 3, 50)
    c = _rand_complex(rng, 50)
    ks = np.meshgrid(*[oracle_mod.mode_range(Ni) for Ni in N[::-1]], indexing="ij")[::-1]
    S = [-k.ravel().astype(np.float64) for k in ks]
    f3 = oracle_mod.direct_type3(X, c, S)
    f1 = oracle_mod.direct_type1(X, c, N).ravel()
    np.testing.assert_allclose(f3, f1, rtol=1e-12, atol=1e-12 * np.abs(f1).max())


def test_direct_type3_bruteforce_loops(oracle_mod):
    rng = _rng(22)
    X = [rng.uniform(-5, 9, 7), rng.uniform(0, 1, 7)]
    S = [rng.uniform(-30, 3, 5), rng.uniform(-2, 2, 5)]
    c = _rand_complex(rng, 7)
    expect = np.array([sum(c[j] * complex(math.cos(S[0][k] * X[0][j] + S[1][k] * X[1][j]),
                                          math.sin(S[0][k] * X[0][j] + S[1][k] * X[1][j])) for j in range(7))
                       for k in range(5)])
    np.testing.assert_allclose(oracle_mod.direct_type3(X, c, S), expect, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle_mod.direct_type3(X, c, S, sel=[4, 1]), expect[[4, 1]], rtol=1e-13, atol=1e-13)


T3_CASES = [(1, 1e-3, 2.0), (1, 1e-9, 2.0), (1, 1e-12, 2.0), (2, 1e-6, 2.0), (2, 1e-12, 2.0), (3, 1e-4, 2.0),
            (3, 1e-9, 2.0), (2, 1e-6, 1.5), (3, 1e-5, 1.25)]


@pytest.mark.parametrize("d,eps,sigma", T3_CASES)
def test_nufft_type3_vs_direct(oracle_mod, d, eps, sigma):
    """The type 3 steps within 10 eps of the exact sum, for point clouds off centre and of widths
    other than 2 pi (sources in [-3, 7)^d, targets in [-20, 5)^d)."""
    rng = _rng(23 + d)
    M, K = 900, 700
    X = [rng.uniform(-3, 7, M) for _ in range(d)]
    S = [rng.uniform(-20, 5, K) for _ in range(d)]
    c = _rand_complex(rng, M)
    f = oracle_mod.nufft_type3(X, c, S, eps, sigma)
    assert oracle_mod.rel_l2(f, oracle_mod.direct_type3(X, c, S)) <= 10 * eps


def test_nufft_type3_degenerate_and_translation(oracle_mod):
    rng = _rng(27)
    eps = 1e-8
    x = [rng.uniform(-1, 1, 300)]
    c = _rand_complex(rng, 300)
    # every target at one frequency; every source at one place; a single target
    for X, S in (([x[0]], [np.full(40, 3.3)]), ([np.full(300, 0.7)], [rng.uniform(-5, 5, 40)]),
                 ([x[0]], [np.array([12.5])])):
        f = oracle_mod.nufft_type3(X, c, S, eps)
        assert oracle_mod.rel_l2(f, oracle_mod.direct_type3(X, c, S)) <= 10 * eps
    # moving every source by a multiplies f_k by exp(i s_k a)
    S = [rng.uniform(-40, 40, 200), rng.uniform(-10, 30, 200)]
    X = [rng.uniform(-2, 2, 300), rng.uniform(0, 3, 300)]
    a = (5.25, -1.5)
    f0 = oracle_mod.nufft_type3(X, c, S, eps)
    f1 = oracle_mod.nufft_type3([X[0] + a[0], X[1] + a[1]], c, S, eps)
    assert oracle_mod.rel_l2(f1, f0 * np.exp(1j * (S[0] * a[0] + S[1] * a[1]))) <= 20 * eps


def test_nufft_clustered_vs_direct(oracle_mod):
    wl = scaled(WORKLOADS["3d_n128_m16m_f32_e5_cluster"], N=(16, 16, 16), M=3000)
    inp = make_inputs(wl)
    f1 = oracle_mod.nufft_type1(inp["X"], inp["c"], wl.N, wl.eps)
    assert oracle_mod.rel_l2(f1, oracle_mod.direct_type1(inp["X"], inp["c"], wl.N)) <= 10 * wl.eps


@pytest.mark.parametrize("N,eps", [((50,), 1e-6), ((20, 24), 1e-6), ((10, 12, 8), 1e-3)])
def test_nufft_type1_type2_adjoint(oracle_mod, N, eps):
    """Steps (7),(9),(10) and (11),(12),interp are exact transposes: adjoint to rounding."""
    rng = _rng(6)
    M = 300
    X = _uniform_points(rng, len(N), M)
    c = _rand_complex(rng, M)
    f = _rand_complex(rng, tuple(reversed(N)))
    lhs = np.vdot(f.ravel(), oracle_mod.nufft_type1(X, c, N, eps).ravel())
    rhs = np.vdot(oracle_mod.nufft_type2(X, f, N, eps), c)
    assert abs(lhs - rhs) <= 1e-13 * abs(lhs)


def test_single_point_closed_form(oracle_mod):
    """M = 1, c = 1: eq. (1) is exp(-i k.x0)."""
    N = (24, 20, 16)
    x0 = [np.array([0.3]), np.array([-2.9]), np.array([1.234])]
    for eps in (1e-3, 1e-6, 1e-10):
        f = oracle_mod.nufft_type1(x0, np.array([1.0 + 0j]), N, eps)
        ks = [oracle_mod.mode_range(Ni) for Ni in N]
        expect = np.exp(-1j * (ks[2][:, None, None] * x0[2][0] + ks[1][None, :, None] * x0[1][0]
                               + ks[0][None, None, :] * x0[0][0]))
        assert oracle_mod.rel_l2(f, expect) <= 10 * eps


def test_single_point_closed_form_1d(oracle_mod):
    """M = 1, c = 1 in 1D: eq. (1) is exp(-i k x0), also for odd N."""
    for N in (32, 33):
        for x0 in (-math.pi, 0.7, math.pi - 1e-9):
            for eps in (1e-2, 1e-5, 1e-12):
                f = oracle_mod.nufft_type1([np.array([x0])], np.array([1.0 + 0j]), (N,), eps)
                expect = np.exp(-1j * oracle_mod.mode_range(N) * x0)
                assert oracle_mod.rel_l2(f, expect) <= 10 * eps


def test_delta_coefficients_closed_form(oracle_mod):
    """f = delta at k0: eq. (3) is exp(i k0.x_j)."""
    rng = _rng(7)
    N = (16, 10)
    X = _uniform_points(rng, 2, 200)
    f = np.zeros((10, 16), complex)
    k0 = (5, -3)
    f[k0[1] + 5, k0[0] + 8] = 1.0
    c = oracle_mod.nufft_type2(X, f, N, 1e-8)
    expect = np.exp(1j * (k0[0] * X[0] + k0[1] * X[1]))
    assert oracle_mod.rel_l2(c, expect) <= 1e-7


def test_translation_by_whole_cells(oracle_mod):
    """Shifting every point by s fine cells shifts the spread grid by s cells, so the NUFFT
    output is multiplied by exp(-i k.s h) (up to rounding of the shifted coordinates)."""
    rng = _rng(8)
    N = (16, 12)
    eps = 1e-9
    prm = oracle_mod.Params(N, eps)
    M = 150
    X = [rng.uniform(-math.pi, 2.0, M) for _ in range(2)]
    c = _rand_complex(rng, M)
    s = (3, 2)
    Xs = [X[i] + s[i] * 2 * math.pi / prm.n[i] for i in range(2)]
    f0 = oracle_mod.nufft_type1(X, c, N, eps)
    f1 = oracle_mod.nufft_type1(Xs, c, N, eps)
    k1 = oracle_mod.mode_range(N[0])[None, :]
    k2 = oracle_mod.mode_range(N[1])[:, None]
    phase = np.exp(-1j * (k1 * s[0] * 2 * math.pi / prm.n[0] + k2 * s[1] * 2 * math.pi / prm.n[1]))
    assert oracle_mod.rel_l2(f1, f0 * phase) <= 1e-12


def test_selected_modes_and_points_match_full(oracle_mod):
    wl = Workload(name="t", dim=3, N=(12, 10, 8), M=500, eps=1e-9, precision="f64", seed=12)
    inp = make_inputs(wl)
    X, c, f = inp["X"], inp["c"], inp["f"]
    full1 = oracle_mod.nufft_type1(X, c, wl.N, wl.eps).ravel()
    sel = np.array([0, 1, 59, 480, 959, 777])
    got = oracle_mod.nufft_type1_at(X, c, wl.N, wl.eps, sel)
    np.testing.assert_allclose(got, full1[sel], rtol=1e-12, atol=1e-12 * np.abs(full1).max())
    full2 = oracle_mod.nufft_type2(X, f, wl.N, wl.eps)
    selp = np.array([4, 0, 499, 250])
    np.testing.assert_allclose(oracle_mod.nufft_type2_at(X, f, wl.N, wl.eps, selp), full2[selp],
                               rtol=1e-14, atol=0)


# ---------------------------------------------------------------------------------------------
# Bin-sort and subproblems (Sec. III-A)
# ---------------------------------------------------------------------------------------------

def test_bins_of_points_at_cell_centres(oracle_mod):
    """Points placed at the centre of known cells land in bin (l1//m1) + nb1 (l2//m2) (+ ...)."""
    n = (24, 20, 12)
    m = (8, 6, 5)
    nb = [(ni + mi - 1) // mi for ni, mi in zip(n, m)]
    rng = _rng(9)
    L = [rng.integers(0, ni, 300) for ni in n]
    X = [-math.pi + (L[i] + 0.5) * 2 * math.pi / n[i] for i in range(3)]
    binv, counts, perm = oracle_mod.binsort(X, n, m)
    expect = (L[0] // m[0]) + nb[0] * ((L[1] // m[1]) + nb[1] * (L[2] // m[2]))
    np.testing.assert_array_equal(binv, expect)
    np.testing.assert_array_equal(counts, np.bincount(expect, minlength=int(np.prod(nb))))
    np.testing.assert_array_equal(perm, np.argsort(expect, kind="stable"))


def test_bins_random_points_cell_interval_and_stable_perm(oracle_mod):
    """For random points, the cell l of the assigned bin satisfies l h <= x + pi < (l + 1) h
    (checked in extended precision), and perm is numpy's stable argsort of the bins."""
    n = (32, 24)
    m = (8, 8)
    rng = _rng(10)
    X = [rng.uniform(-math.pi, math.pi, 5000).astype(np.float32).astype(np.float64) for _ in range(2)]
    binv, counts, perm = oracle_mod.binsort(X, n, m)
    nb0 = (n[0] + m[0] - 1) // m[0]
    b0 = binv % nb0
    b1 = binv // nb0
    for x, bi, ni, mi in ((X[0], b0, n[0], m[0]), (X[1], b1, n[1], m[1])):
        u = (np.longdouble(x) + np.longdouble(math.pi)) * ni / (2 * np.longdouble(math.pi))
        lo = bi * mi
        hi = np.minimum(lo + mi, ni)
        ok = (u >= lo - 1e-9) & (u < hi + 1e-9)
        assert ok.all()
    np.testing.assert_array_equal(counts, np.bincount(binv, minlength=counts.size))
    np.testing.assert_array_equal(perm, np.argsort(binv, kind="stable"))


def test_bins_1d_cell_interval_and_stable_perm(oracle_mod):
    """1D: the bin of a point is floor(l / m) with l h <= x + pi < (l + 1) h, and perm is the
    stable argsort of the bins (a ragged last bin: n not a multiple of m)."""
    n, m = (200,), (32,)
    rng = _rng(12)
    x = rng.uniform(-math.pi, math.pi, 3000).astype(np.float32).astype(np.float64)
    binv, counts, perm = oracle_mod.binsort([x], n, m)
    u = (np.longdouble(x) + np.longdouble(math.pi)) * n[0] / (2 * np.longdouble(math.pi))
    lo = binv * m[0]
    hi = np.minimum(lo + m[0], n[0])
    assert ((u >= lo - 1e-9) & (u < hi + 1e-9)).all()
    assert counts.size == 7
    np.testing.assert_array_equal(counts, np.bincount(binv, minlength=7))
    np.testing.assert_array_equal(perm, np.argsort(binv, kind="stable"))


def test_bins_all_points_in_one_bin(oracle_mod):
    n = (16, 16)
    m = (8, 8)
    X = [np.full(100, -math.pi + 0.1), np.full(100, 0.2)]
    binv, counts, perm = oracle_mod.binsort(X, n, m)
    assert len(set(binv.tolist())) == 1
    assert counts.sum() == 100 and counts.max() == 100
    np.testing.assert_array_equal(perm, np.arange(100))


def test_subproblems_partition(oracle_mod):
    rng = _rng(11)
    counts = rng.integers(0, 50, 40)
    counts[3] = 0
    counts[5] = 200
    cap = 16
    sp = oracle_mod.subproblems(counts, cap)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    # every bin's range is covered exactly once, in order, by chunks of <= cap
    cover = np.zeros(counts.sum(), dtype=int)
    for b, s, ln in sp:
        assert 1 <= ln <= cap
        assert starts[b] <= s and s + ln <= starts[b] + counts[b]
        cover[s:s + ln] += 1
    assert (cover == 1).all()
    assert len(sp) == sum(-(-c // cap) for c in counts)
    assert list(sp[:, 1]) == sorted(sp[:, 1])


def test_points_out_of_range_rejected(oracle_mod):
    X = [np.array([0.0, 20.0]), np.array([0.0, 0.0])]
    with pytest.raises(ValueError):
        oracle_mod.binsort(X, (16, 16), (8, 8))
    with pytest.raises(ValueError):
        oracle_mod.spread([np.array([np.nan]), np.array([0.0])], np.array([1 + 0j]), (16, 16), 4, 9.2)


def test_bins_fold_range_cell_interval(oracle_mod):
    """Coordinates in [pi, 3 pi) and [-3 pi, -pi) fall in the bin of their image in [-pi, pi):
    with u = (x + pi) n / (2 pi) in extended precision and reduced mod n, the bin's cells contain
    u (to 1e-9 cells), and the point lands where the same point shifted by a period lands."""
    n = (40, 24, 18)
    m = (16, 8, 8)
    rng = _rng(13)
    M = 3000
    X = []
    for i in range(3):
        base = rng.uniform(-math.pi, math.pi, M)
        shift = rng.integers(-1, 2, M) * 2 * math.pi
        X.append(np.clip(base + shift, -3 * math.pi, np.nextafter(3 * math.pi, 0)))
    X[0][:4] = [math.pi, -3 * math.pi, np.nextafter(-math.pi, -4.0), 3 * math.pi - 1e-12]
    binv, counts, perm = oracle_mod.binsort(X, n, m)
    nb = [(ni + mi - 1) // mi for ni, mi in zip(n, m)]
    bidx = [binv % nb[0], (binv // nb[0]) % nb[1], binv // (nb[0] * nb[1])]
    for i in range(3):
        u = (np.longdouble(X[i]) + np.longdouble(math.pi)) * n[i] / (2 * np.longdouble(math.pi))
        u = u - n[i] * np.floor(u / n[i])
        lo = bidx[i] * m[i]
        hi = np.minimum(lo + m[i], n[i])
        near_top = u > n[i] - 1e-9        # images that round onto the period's end
        ok = ((u >= lo - 1e-9) & (u < hi + 1e-9)) | (near_top & (hi == n[i]))
        assert ok.all(), i
    np.testing.assert_array_equal(perm, np.argsort(binv, kind="stable"))
    np.testing.assert_array_equal(counts, np.bincount(binv, minlength=int(np.prod(nb))))


@pytest.mark.parametrize("n,w,dist", [((64,), 7, "u"), ((5,), 7, "u"), ((30, 20), 6, "u"), ((7, 9), 13, "u"),
                                      ((16, 12, 10), 6, "u"), ((12, 8, 6), 10, "u"), ((4, 4, 4), 5, "u"),
                                      ((32, 24, 20), 6, "box")])
def test_parallel_spread_interp_equal_serial(oracle_mod, n, w, dist):
    """The parallel spreading (slab-owned) and interpolation (point-parallel) forms return the
    serial loops' results bit for bit, on grids larger and smaller than the kernel, with folded
    coordinates, for any thread count."""
    rng = _rng(17)
    d = len(n)
    M = 2500
    if dist == "box":
        X = [rng.uniform(0.0, 0.5, M) for _ in range(d)]
    else:
        X = [rng.uniform(-math.pi, math.pi, M) for _ in range(d)]
        X[0][:3] = [2.5 * math.pi, -2.9 * math.pi, np.nextafter(-math.pi, -4.0)]
    c = _rand_complex(rng, M)
    beta = 2.30 * w
    ref = oracle_mod.spread(X, c, n, w, beta, threads=1)
    g = _rand_complex(rng, tuple(reversed(n)))
    ref2 = oracle_mod.interp(X, g, w, beta, threads=1)
    for th in (2, 3, 7, 0):
        np.testing.assert_array_equal(oracle_mod.spread(X, c, n, w, beta, threads=th), ref)
        np.testing.assert_array_equal(oracle_mod.interp(X, g, w, beta, threads=th), ref2)
