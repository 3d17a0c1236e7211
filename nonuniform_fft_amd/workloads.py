"""Seeded synthetic workloads for the 1D/2D/3D type 1 / type 2 NUFFT.

This module only draws random inputs and names problem sizes.  It holds none
of the transform's arithmetic, so both the CPU oracle's tests and the GPU path
take their inputs from here without sharing any computation.

The workloads mirror the point distributions of the cuFINUFFT paper
("cuFINUFFT: a load-balanced GPU library for general-purpose nonuniform FFTs",
Sec. IV, task "rand": iid uniform points on the periodic box, density rho of
order one, eq. (16)) at the sizes of the benchmark configurations, plus a
Gaussian-clustered variant that stresses load balance.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "draw_points", "draw_strengths",
           "draw_coefficients", "draw_sparse_coefficients", "scaled"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dim: int
    N: Tuple[int, ...]          # modes per dimension, (N1, N2[, N3]); N1 varies fastest
    M: int                      # number of nonuniform points
    eps: float                  # requested tolerance
    precision: str              # "f32" or "f64"
    dist: str = "uniform"       # "uniform" | "cluster" | "box"
    seed: int = 1000
    cluster_sigma: float = math.pi / 16   # std-dev of each coordinate for dist="cluster"
    box_cells: int = 8                     # dist="box": points iid in [0, box_cells*h)^d

    @property
    def real_dtype(self):
        return np.float32 if self.precision == "f32" else np.float64

    @property
    def complex_dtype(self):
        return np.complex64 if self.precision == "f32" else np.complex128

    @property
    def nmodes(self) -> int:
        return int(np.prod(self.N))


def _w(name, dim, n, M, eps, prec, dist="uniform", seed=1000):
    return Workload(name=name, dim=dim, N=(n,) * dim, M=M, eps=eps, precision=prec, dist=dist,
                    seed=seed)


# Benchmark configurations (sizes, precisions, tolerances and distributions).
WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    _w("2d_n64_m1e4_f32_e5", 2, 64, 10_000, 1e-5, "f32", seed=1001),
    _w("2d_n1024_m4m_f32_e5", 2, 1024, 4_194_304, 1e-5, "f32", seed=1002),
    _w("2d_n1024_m4m_f64_e12", 2, 1024, 4_194_304, 1e-12, "f64", seed=1002),
    _w("3d_n128_m16m_f32_e2", 3, 128, 16_777_216, 1e-2, "f32", seed=1003),
    _w("3d_n128_m16m_f32_e5", 3, 128, 16_777_216, 1e-5, "f32", seed=1003),
    _w("3d_n128_m16m_f32_e5_cluster", 3, 128, 16_777_216, 1e-5, "f32", dist="cluster", seed=1004),
    _w("3d_n256_m134m_f64_e9", 3, 256, 134_217_728, 1e-9, "f64", seed=1005),
    # 1D (the FINUFFT discussion page reports 1D throughputs at tolerance 1e-6 without sizes)
    _w("1d_n1m_m16m_f32_e6", 1, 1 << 20, 1 << 24, 1e-6, "f32", seed=1006),
    _w("1d_n1m_m16m_f64_e6", 1, 1 << 20, 1 << 24, 1e-6, "f64", seed=1006),
]}


def scaled(wl: Workload, N: Optional[Tuple[int, ...]] = None, M: Optional[int] = None,
           **kw) -> Workload:
    """Same distribution/precision at another size (for tests that must finish quickly)."""
    upd = dict(kw)
    if N is not None:
        upd["N"] = tuple(N)
        upd["dim"] = len(N)
    if M is not None:
        upd["M"] = int(M)
    upd.setdefault("name", wl.name + "_scaled")
    return dataclasses.replace(wl, **upd)


def draw_points(wl: Workload, rng: np.random.Generator):
    """Coordinates as a list of d arrays (x, y[, z]) in the workload's real dtype.

    uniform: iid U[-pi, pi).  cluster: iid N(0, sigma^2) per coordinate, folded
    into [-pi, pi).  box: iid uniform in [0, box_cells * 2*pi/n) per coordinate
    with n = 2*N (a tight cluster a few fine cells wide).
    """
    d, M = wl.dim, wl.M
    if wl.dist == "uniform":
        X = rng.uniform(-math.pi, math.pi, size=(d, M))
    elif wl.dist == "cluster":
        X = rng.normal(0.0, wl.cluster_sigma, size=(d, M))
        X = np.mod(X + math.pi, 2 * math.pi) - math.pi
    elif wl.dist == "box":
        X = np.empty((d, M))
        for i in range(d):
            hi = wl.box_cells * 2 * math.pi / (2 * wl.N[i])
            X[i] = rng.uniform(0.0, hi, size=M)
    else:
        raise ValueError(f"unknown distribution {wl.dist!r}")
    X = X.astype(wl.real_dtype)
    return [np.ascontiguousarray(X[i]) for i in range(d)]


def draw_strengths(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    """c_j with real and imaginary parts iid N(0,1), complex dtype of the workload."""
    re = rng.standard_normal(wl.M)
    im = rng.standard_normal(wl.M)
    c = np.empty(wl.M, dtype=wl.complex_dtype)
    c.real = re
    c.imag = im
    return c


def draw_coefficients(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    """f_k with real and imaginary parts iid N(0,1); shape (N3, N2, N1) (N1 fastest)."""
    shape = tuple(reversed(wl.N))
    re = rng.standard_normal(shape)
    im = rng.standard_normal(shape)
    f = np.empty(shape, dtype=wl.complex_dtype)
    f.real = re
    f.imag = im
    return f


def draw_sparse_coefficients(wl: Workload, rng: np.random.Generator, count: int):
    """`count` distinct flat mode positions (k1 fastest) drawn uniformly, with real and imaginary
    parts iid N(0,1): the nonzero entries of an otherwise zero f, for grids too large to fill."""
    total = wl.nmodes
    picks = np.unique(rng.integers(0, total, size=4 * count))[:count]
    while picks.size < count:
        picks = np.unique(np.concatenate([picks, rng.integers(0, total, size=count)]))[:count]
    vals = np.empty(picks.size, dtype=wl.complex_dtype)
    vals.real = rng.standard_normal(picks.size)
    vals.imag = rng.standard_normal(picks.size)
    return picks.astype(np.int64), vals


def make_inputs(wl: Workload, seed: Optional[int] = None, want_c: bool = True,
                want_f: bool = True, sparse_f: int = 0):
    """Points, then strengths, then coefficients, from one PCG64 stream.  With sparse_f > 0 the
    coefficients are that many nonzero modes ("f_modes", "f_vals") instead of a dense "f"."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    out = {"X": draw_points(wl, rng)}
    if want_c:
        out["c"] = draw_strengths(wl, rng)
    if sparse_f > 0:
        out["f_modes"], out["f_vals"] = draw_sparse_coefficients(wl, rng, sparse_f)
    elif want_f:
        out["f"] = draw_coefficients(wl, rng)
    return out
