"""Helpers for the GPU parity tests: run the HIP path on numpy inputs, compare with the oracle."""
import numpy as np

try:
    import torch
except Exception:  # pragma: no cover
    torch = None


def dev():
    return torch.device("cuda", 0)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def cdtype(prec):
    return torch.complex64 if prec == "f32" else torch.complex128


def make_plan(nf, nufft_type, N, eps, prec, **kw):
    return nf.Plan(nufft_type, N, eps, prec, **kw)


def gpu_type1(nf, X, c, N, eps, prec, **kw):
    p = make_plan(nf, 1, N, eps, prec, **kw)
    p.setpts(*[to_dev(x) for x in X])
    f = torch.empty(tuple(reversed(tuple(N))), dtype=cdtype(prec), device=dev())
    p.execute(to_dev(c) if len(c) else torch.empty(0, dtype=cdtype(prec), device=dev()), f)
    torch.cuda.synchronize()
    out = f.cpu().numpy()
    p.destroy()
    return out


def gpu_type2(nf, X, f, N, eps, prec, **kw):
    p = make_plan(nf, 2, N, eps, prec, **kw)
    p.setpts(*[to_dev(x) for x in X])
    M = len(X[0])
    c = torch.empty(M, dtype=cdtype(prec), device=dev())
    p.execute(c, to_dev(f))
    torch.cuda.synchronize()
    out = c.cpu().numpy()
    p.destroy()
    return out


def tol_for(prec):
    """Parity bar against the oracle NUFFT: relative l2 1e-5 (fp32), 1e-10 (fp64)."""
    return 1e-5 if prec == "f32" else 1e-10
