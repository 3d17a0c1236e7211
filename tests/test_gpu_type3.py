"""Type 3 on the GPU (nufft_setpts_type3 + nufft_execute) against the oracle's type 3 steps, to
1e-5 (fp32) / 1e-10 (fp64), and against the exact sum within 10 eps.  Sources and targets are
off centre, of widths other than 2 pi, and include the degenerate clouds (all targets at one
frequency, all sources at one place) and empty inputs."""
import math
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

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


def _cloud(rng, d, M, K, prec, xr=(-3.0, 7.0), sr=(-20.0, 5.0)):
    rd = np.float32 if prec == "f32" else np.float64
    X = [rng.uniform(*xr, M).astype(rd) for _ in range(d)]
    S = [rng.uniform(*sr, K).astype(rd) for _ in range(d)]
    c = (rng.standard_normal(M) + 1j * rng.standard_normal(M)).astype(np.complex64 if prec == "f32" else np.complex128)
    return X, S, c


def _gpu_t3(nf, X, S, c, eps, prec, **kw):
    d = len(X)
    p = nf.Plan(3, d, eps, prec, **kw)
    p.setpts_type3([to_dev(x) for x in X], [to_dev(s) for s in S])
    f = torch.empty(len(S[0]), dtype=cdtype(prec), device=dev())
    p.execute(to_dev(c) if len(c) else torch.empty(0, dtype=cdtype(prec), device=dev()), f)
    torch.cuda.synchronize()
    n = p.n
    p.destroy()
    return f.cpu().numpy(), n


CASES = [(1, 30_001, 20_000, 1e-5, "f32"), (1, 20_000, 9_999, 1e-12, "f64"), (2, 40_000, 30_000, 1e-5, "f32"),
         (2, 20_000, 20_000, 1e-10, "f64"), (3, 40_000, 30_000, 1e-4, "f32"), (3, 40_000, 30_000, 1e-5, "f32"),
         (3, 15_000, 12_000, 1e-9, "f64")]


def _t3_tol(prm, prec):
    """Bar against the fp64 oracle.  A single-precision plan stores the scaled sources
    y = (x - C) / gamma and targets theta = (s - D) gamma h in fp32 (unit roundoff u = 2^-24):
      * |y| <= X / gamma, so the phase xi y of a source term (|xi| <= S gamma) moves by at most
        u X S;
      * |theta| <= S gamma h = pi / sigma, and the inner type 2 sums modes |k| <= n / 2, so a target's
        phase k theta moves by at most u pi n / (2 sigma).
    Phase errors add over dimensions, and the output's relative l2 error is at most their largest
    value (about its rms for incoherent sums).  Bar: max(1e-5 fp32 / 1e-10 fp64, 2 u sum_i
    (X_i S_i + pi n_i / (2 sigma))); for fp64 plans the rounding term is negligible."""
    u = 2.0 ** -24 if prec == "f32" else 2.0 ** -53
    phase = sum(Xi * Si + math.pi * ni / (2 * prm.sigma) for Xi, Si, ni in zip(prm.X, prm.S, prm.n))
    return max(tol_for(prec), 2 * u * phase)


@pytest.mark.parametrize("d,M,K,eps,prec", CASES)
@pytest.mark.parametrize("method", [0, 1], ids=["auto", "GMsort"])
def test_type3_vs_oracle(nf, orc, d, M, K, eps, prec, method):
    print(f"type3 d={d} M={M} K={K} eps={eps} {prec} method={method}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(100 + d)
    X, S, c = _cloud(rng, d, M, K, prec)
    f, n = _gpu_t3(nf, X, S, c, eps, prec, method=method)
    prm = orc.Type3Params(X, S, eps)
    assert n == prm.n
    ref = orc.nufft_type3(X, c, S, eps)
    err = orc.rel_l2(f, ref)
    assert err <= _t3_tol(prm, prec), (err, _t3_tol(prm, prec))
    sel = np.sort(rng.choice(K, 64, replace=False))
    exact = orc.direct_type3(X, c, S, sel=sel)
    assert orc.rel_l2(f[sel], exact) <= 10 * eps


def test_type3_degenerate_and_empty(nf, orc):
    rng = np.random.default_rng(7)
    eps = 1e-9
    x = rng.uniform(-1, 1, 3000)
    c = rng.standard_normal(3000) + 1j * rng.standard_normal(3000)
    for X, S in (([x], [np.full(40, 3.3)]), ([np.full(3000, 0.7)], [rng.uniform(-5, 5, 40)]),
                 ([x], [np.array([12.5])]), ([x, x[::-1].copy()], [rng.uniform(-9, 9, 77), np.zeros(77)])):
        f, _ = _gpu_t3(nf, X, S, c, eps, "f64")
        assert orc.rel_l2(f, orc.direct_type3(X, c, S)) <= 10 * eps
    # no sources: f = 0; no targets: nothing written
    f, _ = _gpu_t3(nf, [np.zeros(0)], [rng.uniform(-3, 3, 9)], np.zeros(0, complex), eps, "f64")
    assert not f.any()
    f, _ = _gpu_t3(nf, [x], [np.zeros(0)], c, eps, "f64")
    assert f.size == 0


def test_type3_errors(nf):
    p = nf.Plan(3, 2, 1e-6, "f64")
    x = to_dev(np.array([0.0, np.nan]))
    with pytest.raises(nf.NufftError) as ei:
        p.setpts_type3([x, x], [x, x])
    assert ei.value.code == -6
    q = nf.Plan(1, (16, 16), 1e-6, "f64")
    lib = nf.load_library()
    assert lib.nufft_setpts_type3(q.handle, 0, None, None, None, 0, None, None, None) == -1
    p.setpts_type3([to_dev(np.zeros(3))] * 2, [to_dev(np.zeros(2))] * 2)
    c = torch.zeros(3, dtype=torch.complex128, device=dev())
    f = torch.zeros(2, dtype=torch.complex128, device=dev())
    import ctypes
    assert lib.nufft_execute_adjoint(p.handle, ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(f.data_ptr())) == -7
    p.destroy()
    q.destroy()
