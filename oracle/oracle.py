"""Plain CPU oracle for the 1D/2D/3D type 1 and type 2 NUFFT (fp64).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library.  It shares no code
with the GPU path.

Source of every step: "cuFINUFFT: a load-balanced GPU library for
general-purpose nonuniform FFTs" (Shih, Wright, Anden, Blaschke, Barnett):
  * eqs. (1)-(3): type 1 / type 2 exact sums and the mode set I_N;
  * eq. (4): Fourier transform convention; eq. (5): the ES kernel;
  * eq. (6): kernel width w and shape beta from the tolerance, fine grid n;
  * eqs. (7)-(10): type 1 = spread, plain FFT, truncate + correct;
  * eqs. (11)-(12) and the interpolation sum after them: type 2;
  * Sec. III-A: bins, the "inside a bin" rule and subproblems.
The tolerance-to-width table on "CUFINUFFT binsize and performance"
(flatironinstitute/finufft discussion #809, section "Tolerance (Kernel Width
ns)") pins eq. (6)'s width rule.

Readings taken where the pages are silent or garbled (all listed in the
design notes): beta = 2.30 w (the digits after "2." are lost); exact powers of
ten map to the integer log; w is clamped to [2, 16]; grid cell l sits at
l h - pi (the bin rule's origin), which multiplies the correction by (-1)^k;
the correction is (2/w)^d / prod_i phihat(alpha_i k_i); phihat is computed by
quadrature of eq. (4); modes are stored k1 fastest, each k_i ascending from
-floor(N_i/2).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import List, Optional, Sequence, Tuple

import numpy as np
import scipy.fft

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nufft_oracle.c")
_LIBDIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIBDIR, "libnufft_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the C part of the oracle with gcc (fp64, no FP contraction, no fast-math)."""
    os.makedirs(_LIBDIR, exist_ok=True)
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
               "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_int64
        D = ctypes.c_double
        lib.oracle_grid_scale.argtypes = [L]
        lib.oracle_grid_scale.restype = D
        lib.oracle_es_kernel.argtypes = [D, D]
        lib.oracle_es_kernel.restype = D
        for name in ("oracle_spread", "oracle_interp"):
            fn = getattr(lib, name)
            fn.argtypes = [I, P, I, D, L, P, P, P]
            fn.restype = I
        for name in ("oracle_spread_par", "oracle_interp_par"):
            fn = getattr(lib, name)
            fn.argtypes = [I, P, I, D, L, P, P, P, I]
            fn.restype = I
        lib.oracle_binsort.argtypes = [I, P, P, L, P, P, P, P]
        lib.oracle_binsort.restype = I
        lib.oracle_subproblems.argtypes = [L, P, L, P]
        lib.oracle_subproblems.restype = L
        for name in ("oracle_direct_type1", "oracle_direct_type2"):
            fn = getattr(lib, name)
            fn.argtypes = [I, P, L, P, P, L, P, P]
            fn.restype = I
        lib.oracle_type1_bhat_at.argtypes = [I, P, I, D, L, P, P, L, P, P]
        lib.oracle_type1_bhat_at.restype = I
        _lib = lib
    return _lib


# ----------------------------------------------------------------------------------------------
# Plan parameters (eq. (6)) and correction factors (eqs. (4), (5), (10))
# ----------------------------------------------------------------------------------------------

BETA_OVER_W = 2.30
W_MIN, W_MAX = 2, 16


# Upsampling factors other than 2 (the page fixes sigma = 2 and names smaller ones as future work,
# Sec. I-B item (3)).  Reading: the kernel's Fourier transform must have decayed where the first
# alias of the band, xi = alpha (n - N/2) = w pi (1 - 1/(2 sigma)), starts, so
# beta = GAMMA pi (1 - 1/(2 sigma)) w, with GAMMA fixed by the page's beta = 2.30 w at sigma = 2;
# the error of the truncated kernel falls like exp(-pi w sqrt(1 - 1/sigma)), so
# w = ceil(ln(1/eps) / (pi sqrt(1 - 1/sigma))), which reproduces the page's width table at sigma = 2.
SIGMA_MIN, SIGMA_MAX = 1.25, 2.0
GAMMA = BETA_OVER_W / (0.75 * math.pi)


def kernel_params(eps: float, sigma: float = 2.0) -> Tuple[int, float]:
    """Eq. (6): w = ceil(log10(1/eps)) + 1 (values within 1e-9 of an integer count as it),
    clamped to [2, 16]; beta = 2.30 * w.  For sigma < 2 the rule of the reading above."""
    if not (eps > 0):
        raise ValueError("eps must be positive")
    if not (SIGMA_MIN <= sigma <= SIGMA_MAX):
        raise ValueError("sigma must be in [1.25, 2]")
    if sigma == 2.0:
        w = int(math.ceil(math.log10(1.0 / eps) - 1e-9)) + 1
        w = max(W_MIN, min(W_MAX, w))
        return w, BETA_OVER_W * w
    w = int(math.ceil(math.log(1.0 / eps) / (math.pi * math.sqrt(1.0 - 1.0 / sigma)) - 1e-9))
    w = max(W_MIN, min(W_MAX, w))
    return w, GAMMA * math.pi * (1.0 - 0.5 / sigma) * w


def _is_5smooth(v: int) -> bool:
    for p in (2, 3, 5):
        while v % p == 0:
            v //= p
    return v == 1


def fine_size(N: int, w: int, sigma: float = 2.0) -> int:
    """Sec. II: smallest 2^q 3^p 5^r that is >= max(sigma*N, w) (sigma N rounded up)."""
    v = max(int(math.ceil(sigma * int(N) - 1e-9)), int(w), 1)
    while not _is_5smooth(v):
        v += 1
    return v


def phihat(xi, w: int, beta: float, nodes: int = 200) -> np.ndarray:
    """Fourier transform of the ES kernel, eq. (4) applied to eq. (5):
        phihat(xi) = int_{-1}^{1} exp(beta (sqrt(1-z^2) - 1)) cos(xi z) dz
    (the kernel is even, so only the cosine part survives).  Substituting
    z = sin(theta) removes the square-root endpoint behaviour,
        = int_{-pi/2}^{pi/2} exp(beta (cos(theta) - 1)) cos(xi sin(theta)) cos(theta) dtheta,
    which Gauss-Legendre quadrature (numpy's nodes) integrates to rounding level."""
    del w  # the kernel depends on w only through beta and the scaling alpha
    xi = np.asarray(xi, dtype=np.float64)
    g, wt = np.polynomial.legendre.leggauss(nodes)
    th = 0.5 * math.pi * g
    wt = 0.5 * math.pi * wt
    base = np.exp(beta * (np.cos(th) - 1.0)) * np.cos(th) * wt
    return np.cos(np.multiply.outer(xi, np.sin(th))) @ base


def mode_range(N: int) -> np.ndarray:
    """I_N of eq. (2): integers k with -N/2 <= k < N/2, ascending."""
    return np.arange(-(N // 2), N - N // 2, dtype=np.int64)


def correction_1d(N: int, n: int, w: int, beta: float) -> np.ndarray:
    """Per-dimension correction factor of eq. (10), for k in I_N:
        p(k) = (h / alpha) (-1)^k / phihat(alpha k),  h/alpha = 2/w,  alpha = w pi / n.
    The (-1)^k is the phase of the grid origin at -pi (the bin rule's origin)."""
    k = mode_range(N)
    alpha = w * math.pi / n
    sign = np.where(k % 2 == 0, 1.0, -1.0)
    return (2.0 / w) * sign / phihat(alpha * k, w, beta)


class Params:
    """Everything the algorithm fixes from (d, N, eps) and the bin geometry."""

    def __init__(self, N: Sequence[int], eps: float, sigma: float = 2.0):
        self.N = tuple(int(v) for v in N)
        self.dim = len(self.N)
        if self.dim not in (1, 2, 3):
            raise ValueError("dimension must be 1, 2 or 3")
        self.eps = float(eps)
        self.sigma = float(sigma)
        self.w, self.beta = kernel_params(eps, self.sigma)
        self.n = tuple(fine_size(Ni, self.w, self.sigma) for Ni in self.N)
        self.p = [correction_1d(Ni, ni, self.w, self.beta) for Ni, ni in zip(self.N, self.n)]


# ----------------------------------------------------------------------------------------------
# Marshalling helpers
# ----------------------------------------------------------------------------------------------

def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _c128_interleaved(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.complex128).reshape(-1)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _coords(X) -> Tuple[List[np.ndarray], ctypes.Array]:
    xs = [_f64(x) for x in X]
    arr = (ctypes.c_void_p * 3)(*([x.ctypes.data for x in xs] + [None] * (3 - len(xs))))
    return xs, arr


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.int64)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"{what} failed with code {rc} (bad argument or point out of range)")


# ----------------------------------------------------------------------------------------------
# Steps of the method
# ----------------------------------------------------------------------------------------------

# Threads of the parallel spreading / interpolation forms (0 = all host cores, 1 = the plain serial
# loops).  The parallel forms return the serial results bit for bit (slab-owned spreading, one
# independent sum per point); the CPU-baseline timing sets 1 for its serial leg.
THREADS = 0


def spread(X, c, n: Sequence[int], w: int, beta: float, threads: Optional[int] = None) -> np.ndarray:
    """Type 1 step 1, eq. (7).  Returns b with shape (n3, n2, n1) (n1 fastest), complex128."""
    lib = _load()
    d = len(n)
    xs, xa = _coords(X)
    cc = _c128_interleaved(c)
    M = xs[0].size
    b = np.zeros(int(np.prod(n)), dtype=np.complex128)
    nn = _i64(n)
    th = THREADS if threads is None else threads
    if th == 1:
        rc = lib.oracle_spread(d, _ptr(nn), w, beta, M, xa, _ptr(cc), _ptr(b))
    else:
        rc = lib.oracle_spread_par(d, _ptr(nn), w, beta, M, xa, _ptr(cc), _ptr(b), th)
    _check(rc, "spread")
    return b.reshape(tuple(reversed(n)))


def interp(X, b, w: int, beta: float, threads: Optional[int] = None) -> np.ndarray:
    """Type 2 step 3 (interpolation sum after eq. (12)).  b has shape (n3, n2, n1)."""
    lib = _load()
    b = np.asarray(b)
    n = tuple(reversed(b.shape))
    d = len(n)
    xs, xa = _coords(X)
    bb = _c128_interleaved(b)
    M = xs[0].size
    c = np.zeros(M, dtype=np.complex128)
    nn = _i64(n)
    th = THREADS if threads is None else threads
    if th == 1:
        rc = lib.oracle_interp(d, _ptr(nn), w, beta, M, xa, _ptr(bb), _ptr(c))
    else:
        rc = lib.oracle_interp_par(d, _ptr(nn), w, beta, M, xa, _ptr(bb), _ptr(c), th)
    _check(rc, "interp")
    return c


# Threads the library FFT may use (-1 = all host cores).  The CPU-baseline timing sets 1.
FFT_WORKERS = -1


def fft_forward(b: np.ndarray) -> np.ndarray:
    """Eq. (9): bhat_k = sum_l b_l exp(-2 pi i l.k/n), unnormalised (library FFT)."""
    return scipy.fft.fftn(b, workers=FFT_WORKERS)


def fft_backward(bhat: np.ndarray) -> np.ndarray:
    """Eq. (12): b_l = sum_k bhat_k exp(+2 pi i l.k/n), unnormalised (library FFT)."""
    return scipy.fft.ifftn(bhat, norm="forward", workers=FFT_WORKERS)


def _index_grids(N, n):
    """Fine-grid positions k mod n of every mode k in I_N, per dimension (arrays in slow..fast order)."""
    return [mode_range(Ni) % ni for Ni, ni in zip(N, n)][::-1]


def _outer_p(p_list) -> np.ndarray:
    """Tensor product p(k) = prod_i p_i(k_i), shaped (N3, N2, N1)."""
    out = np.array(1.0)
    for p in p_list[::-1]:
        out = np.multiply.outer(out, p)
    return out


def truncate_correct(bhat: np.ndarray, prm: Params) -> np.ndarray:
    """Type 1 step 3, eq. (10): f_k = p_k bhat_{k mod n} for k in I_N; shape (N3, N2, N1)."""
    idx = _index_grids(prm.N, prm.n)
    return _outer_p(prm.p) * bhat[np.ix_(*idx)]


def precorrect_pad(f: np.ndarray, prm: Params) -> np.ndarray:
    """Type 2 step 1, eq. (11): bhat_{k mod n} = p_k f_k on I_N, zero elsewhere on I_n."""
    bhat = np.zeros(tuple(reversed(prm.n)), dtype=np.complex128)
    idx = _index_grids(prm.N, prm.n)
    bhat[np.ix_(*idx)] = _outer_p(prm.p) * np.asarray(f, dtype=np.complex128).reshape(
        tuple(reversed(prm.N)))
    return bhat


def nufft_type1(X, c, N: Sequence[int], eps: float, sigma: float = 2.0) -> np.ndarray:
    """Approximate eq. (1) by eqs. (7), (9), (10).  Returns f with shape (N3, N2, N1)."""
    prm = Params(N, eps, sigma)
    b = spread(X, c, prm.n, prm.w, prm.beta)
    return truncate_correct(fft_forward(b), prm)


def type2_grid(f, N: Sequence[int], eps: float, sigma: float = 2.0):
    """Type 2 steps 1-2 (eqs. (11), (12)): the fine grid b that step 3 interpolates from."""
    prm = Params(N, eps, sigma)
    return fft_backward(precorrect_pad(f, prm)), prm


def nufft_type2(X, f, N: Sequence[int], eps: float, sigma: float = 2.0) -> np.ndarray:
    """Approximate eq. (3) by eqs. (11), (12) and the interpolation sum.  Returns c (M,)."""
    b, prm = type2_grid(f, N, eps, sigma)
    return interp(X, b, prm.w, prm.beta)


def nufft_type2_at(X, f, N: Sequence[int], eps: float, sel: Sequence[int]) -> np.ndarray:
    """Type 2 at the points listed in `sel` only (the grid is still built in full)."""
    b, prm = type2_grid(f, N, eps)
    sel = np.asarray(sel, dtype=np.int64)
    return interp([np.asarray(x)[sel] for x in X], b, prm.w, prm.beta)


def nufft_type1_at(X, c, N: Sequence[int], eps: float, sel: Sequence[int]) -> np.ndarray:
    """Type 1 at the flat output positions listed in `sel` (k1 fastest), without forming
    the whole fine grid: eq. (9) at those k with eq. (7) inserted (see the C routine),
    then the correction of eq. (10)."""
    lib = _load()
    prm = Params(N, eps)
    d = prm.dim
    sel = np.asarray(sel, dtype=np.int64)
    # positions -> (k1, k2[, k3]) and the correction factor at each
    kv = np.empty((sel.size, d), dtype=np.int64)
    pk = np.ones(sel.size)
    rem = sel.copy()
    for i in range(d):
        pos_i = rem % prm.N[i]
        rem = rem // prm.N[i]
        kv[:, i] = pos_i - prm.N[i] // 2
        pk = pk * prm.p[i][pos_i]
    xs, xa = _coords(X)
    cc = _c128_interleaved(c)
    out = np.zeros(sel.size, dtype=np.complex128)
    nn = _i64(prm.n)
    kv = np.ascontiguousarray(kv)
    _check(lib.oracle_type1_bhat_at(d, _ptr(nn), prm.w, prm.beta, xs[0].size, xa, _ptr(cc),
                                    sel.size, _ptr(kv), _ptr(out)), "type1_bhat_at")
    return pk * out


# ----------------------------------------------------------------------------------------------
# Exact sums (eqs. (1), (3))
# ----------------------------------------------------------------------------------------------

def direct_type1(X, c, N: Sequence[int], sel: Optional[Sequence[int]] = None) -> np.ndarray:
    """Eq. (1) summed term by term.  Without `sel` returns shape (N3, N2, N1); with `sel`
    (flat output positions, k1 fastest) returns those entries only."""
    lib = _load()
    d = len(N)
    xs, xa = _coords(X)
    cc = _c128_interleaved(c)
    NN = _i64(N)
    if sel is None:
        out = np.zeros(int(np.prod(N)), dtype=np.complex128)
        _check(lib.oracle_direct_type1(d, _ptr(NN), xs[0].size, xa, _ptr(cc), 0, None, _ptr(out)),
               "direct_type1")
        return out.reshape(tuple(reversed(tuple(N))))
    s = _i64(sel)
    out = np.zeros(s.size, dtype=np.complex128)
    _check(lib.oracle_direct_type1(d, _ptr(NN), xs[0].size, xa, _ptr(cc), s.size, _ptr(s),
                                   _ptr(out)), "direct_type1")
    return out


def direct_type2(X, f, N: Sequence[int], sel: Optional[Sequence[int]] = None) -> np.ndarray:
    """Eq. (3) summed term by term, at all points or at the point indices in `sel`."""
    lib = _load()
    d = len(N)
    xs, xa = _coords(X)
    ff = _c128_interleaved(f)
    NN = _i64(N)
    M = xs[0].size
    if sel is None:
        out = np.zeros(M, dtype=np.complex128)
        _check(lib.oracle_direct_type2(d, _ptr(NN), M, xa, _ptr(ff), 0, None, _ptr(out)),
               "direct_type2")
        return out
    s = _i64(sel)
    out = np.zeros(s.size, dtype=np.complex128)
    _check(lib.oracle_direct_type2(d, _ptr(NN), M, xa, _ptr(ff), s.size, _ptr(s), _ptr(out)),
           "direct_type2")
    return out


def direct_type2_modes(X, N: Sequence[int], modes: Sequence[int], vals) -> np.ndarray:
    """Eq. (3) summed term by term over the nonzero coefficients only: f is zero except at the
    flat mode positions `modes` (k1 fastest, k_i in I_N of eq. (2)), where it holds `vals`.
    Returns c at every point."""
    d = len(N)
    modes = np.asarray(modes, dtype=np.int64)
    vals = np.asarray(vals, dtype=np.complex128)
    # the mode vector of each flat position
    ks = []
    rest = modes.copy()
    for i in range(d):
        ks.append(mode_range(int(N[i]))[rest % int(N[i])].astype(np.float64))
        rest //= int(N[i])
    M = np.asarray(X[0]).size
    out = np.zeros(M, dtype=np.complex128)
    for lo in range(0, M, 4096):
        ph = np.zeros((min(M, lo + 4096) - lo, modes.size))
        for i in range(d):
            ph += np.outer(np.asarray(X[i], dtype=np.float64)[lo:lo + 4096], ks[i])
        out[lo:lo + ph.shape[0]] = np.exp(1j * ph) @ vals
    return out


# ----------------------------------------------------------------------------------------------
# Bin-sort and subproblems (Sec. III-A)
# ----------------------------------------------------------------------------------------------

# ----------------------------------------------------------------------------------------------
# Type 3, nonuniform to nonuniform: f_k = sum_j c_j exp(+i s_k . x_j).  The cuFINUFFT page lists
# it as not provided (Sec. I-B, item 4); the imaging equation of the GPU training page ("A toy
# problem": irregular visibility samples to image points) is a sum of this class.  The steps
# below are a reading built from the type 1 and type 2 steps of Sec. II:
#   1. centre and half-width per dimension: sources x in C +- X, targets s in D +- S;
#   2. fine grid n (smallest even 5-smooth >= max(2 sigma X S / pi + w, 2 w)), h = 2 pi / n and
#      scale gamma = n / (2 sigma S): the scaled sources y = (x - C) / gamma keep the kernel's
#      reach inside [-pi, pi), and the scaled targets xi = (s - D) gamma stay inside the band
#      |xi h| <= pi / sigma that the kernel resolves (as the modes of type 1 do);
#   3. c'_j = c_j exp(i D.(x_j - C)); spread c' at y onto the grid (eq. (7));
#   4. sum_l b_l exp(i xi t_l) over cells t_l = l h - pi is a type 2 sum with N = n modes
#      (f_k = b_{k + floor(n/2)}) at points theta = xi h, evaluated by the type 2 NUFFT;
#   5. divide by the kernel transform, sum_l psi(t_l - y) exp(i xi t_l) ~ (1/h) psihat(xi)
#      exp(i xi y) with psihat(xi) = alpha phihat(alpha xi), alpha = w h / 2, i.e. multiply by
#      prod_i (2/w) / phihat(alpha_i xi_i), and restore the phases exp(i s.C) and
#      exp(i xi (h floor(n/2) - pi)).
# ----------------------------------------------------------------------------------------------

def _even_5smooth(v: float) -> int:
    u = max(int(math.ceil(v - 1e-9)), 2)
    while u % 2 or not _is_5smooth(u):
        u += 1
    return u


class Type3Params:
    """Centres, half-widths, fine grid, scales and kernel of a type 3 transform (steps 1, 2)."""

    def __init__(self, X, S, eps: float, sigma: float = 2.0):
        self.dim = len(X)
        self.w, self.beta = kernel_params(eps, sigma)
        self.sigma = float(sigma)
        xs = [np.asarray(x, dtype=np.float64) for x in X]
        ss = [np.asarray(s, dtype=np.float64) for s in S]
        self.C = [0.5 * (x.max() + x.min()) if x.size else 0.0 for x in xs]
        self.X = [0.5 * (x.max() - x.min()) if x.size else 0.0 for x in xs]
        self.D = [0.5 * (s.max() + s.min()) if s.size else 0.0 for s in ss]
        self.S = [0.5 * (s.max() - s.min()) if s.size else 0.0 for s in ss]
        w = self.w
        self.n = tuple(_even_5smooth(max(2 * sigma * Xi * Si / math.pi + w, 2 * w)) for Xi, Si in zip(self.X, self.S))
        self.h = [2 * math.pi / ni for ni in self.n]
        self.gamma = []
        for Xi, Si, ni in zip(self.X, self.S, self.n):
            if Si > 0:
                self.gamma.append(ni / (2 * sigma * Si))
            elif Xi > 0:
                self.gamma.append(Xi * ni / (math.pi * (ni - w)))
            else:
                self.gamma.append(1.0)


def nufft_type3(X, c, S, eps: float, sigma: float = 2.0) -> np.ndarray:
    """Type 3 by the steps above, all in fp64: f_k ~ sum_j c_j exp(+i s_k . x_j), k = 1..K."""
    prm = Type3Params(X, S, eps, sigma)
    xs = [np.asarray(x, dtype=np.float64) for x in X]
    ss = [np.asarray(s, dtype=np.float64) for s in S]
    y = [(x - Ci) / g for x, Ci, g in zip(xs, prm.C, prm.gamma)]
    pre = np.zeros(xs[0].size)
    for x, Ci, Di in zip(xs, prm.C, prm.D):
        pre = pre + Di * (x - Ci)
    cp = np.asarray(c, dtype=np.complex128) * np.exp(1j * pre)
    b = spread(y, cp, prm.n, prm.w, prm.beta)
    theta = [(s - Di) * g * hi for s, Di, g, hi in zip(ss, prm.D, prm.gamma, prm.h)]
    cin = nufft_type2(theta, b, prm.n, eps, sigma)
    out = cin.astype(np.complex128)
    for s, Ci, Di, g, hi, ni in zip(ss, prm.C, prm.D, prm.gamma, prm.h, prm.n):
        xi = (s - Di) * g
        alpha = prm.w * hi / 2
        out = out * (2.0 / prm.w) / phihat(alpha * xi, prm.w, prm.beta)
        out = out * np.exp(1j * (xi * (hi * (ni // 2) - math.pi) + s * Ci))
    return out


def direct_type3(X, c, S, sel: Optional[Sequence[int]] = None) -> np.ndarray:
    """The exact type 3 sum f_k = sum_j c_j exp(+i s_k . x_j) in fp64 (targets in chunks); `sel`
    restricts it to the listed targets."""
    xs = [np.asarray(x, dtype=np.float64) for x in X]
    ss = [np.asarray(s, dtype=np.float64) for s in S]
    if sel is not None:
        sel = np.asarray(sel, dtype=np.int64)
        ss = [s[sel] for s in ss]
    cc = np.asarray(c, dtype=np.complex128)
    K = ss[0].size
    out = np.zeros(K, dtype=np.complex128)
    step = max(1, (1 << 22) // max(1, xs[0].size))
    for a in range(0, K, step):
        ph = np.zeros((min(K, a + step) - a, xs[0].size))
        for s, x in zip(ss, xs):
            ph += np.multiply.outer(s[a:a + step], x)
        out[a:a + step] = np.exp(1j * ph) @ cc
    return out


def binsort(X, n: Sequence[int], m: Sequence[int]):
    """Returns (bin_of_point, counts, perm) as int64 arrays: bins x-fastest (Sec. III-A), perm the
    points read out bin by bin, increasing original index inside a bin (see the C routine)."""
    lib = _load()
    d = len(n)
    xs, xa = _coords(X)
    M = xs[0].size
    nb = [(ni + mi - 1) // mi for ni, mi in zip(n, m)]
    nbins = int(np.prod(nb))
    binv = np.zeros(M, dtype=np.int64)
    counts = np.zeros(nbins, dtype=np.int64)
    perm = np.zeros(M, dtype=np.int64)
    nn, mm = _i64(n), _i64(m)
    _check(lib.oracle_binsort(d, _ptr(nn), _ptr(mm), M, xa, _ptr(binv), _ptr(counts), _ptr(perm)), "binsort")
    return binv, counts, perm


def subproblems(counts, cap: int) -> np.ndarray:
    """(bin, start, length) rows: each bin's sorted points in chunks of at most `cap`."""
    lib = _load()
    cnt = _i64(counts)
    ns = lib.oracle_subproblems(cnt.size, _ptr(cnt), int(cap), None)
    if ns < 0:
        raise ValueError("bad subproblem cap")
    out = np.zeros((max(ns, 0), 3), dtype=np.int64)
    if ns > 0:
        lib.oracle_subproblems(cnt.size, _ptr(cnt), int(cap), _ptr(out))
    return out


def grid_scale(n: int) -> float:
    """s = n / (2 pi) as the oracle rounds it."""
    return _load().oracle_grid_scale(int(n))


def es_kernel(z: float, beta: float) -> float:
    return _load().oracle_es_kernel(float(z), float(beta))


def rel_l2(a, b) -> float:
    """Relative l2 error ||a - b|| / ||b|| over all entries (complex promoted to fp64)."""
    a = np.asarray(a, dtype=np.complex128).ravel()
    b = np.asarray(b, dtype=np.complex128).ravel()
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))
