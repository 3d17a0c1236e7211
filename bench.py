#!/usr/bin/env python3
"""Benchmark of the 3D type 1 + type 2 NUFFT on one MI355X.

One step = the whole hot path over one batch of points: bin-sort (setpts), type 1
(clear, spread, FFT, deconvolve) and type 2 on the same sorted points (pre-correct/pad,
FFT, interpolate), for the 3D fp32 eps = 1e-5 workload (N = 128^3 modes, M = 2^24 iid
uniform points, complex Gaussian strengths and coefficients).  Inputs are resident in
HBM before timing starts.  `value` is NU points per second through the type-1 + type-2
pair including the sort (M / step time).

Prints ONE JSON line.  Extra fields give per-type exec-only throughput, per-stage times,
the roofline of the dominant kernel and the CPU-oracle baseline.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth


def spread_bytes(M, dim, n, real_size):
    """Algorithmic bytes of one spread (or interp) launch: sorted coordinates, permutation,
    strengths gather, one pass over the fine grid: M (d s + 2 s + 4) + prod(n) 2 s."""
    cells = 1
    for v in n:
        cells *= v
    return M * (dim * real_size + 2 * real_size + 4) + cells * 2 * real_size


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_pair(orc, wl, X, c, f):
    """The oracle's bin-sort, type 1 (spread, FFT, correct) and type 2 (pad, inverse FFT,
    interpolate) on the given points; per-stage seconds."""
    prm = orc.Params(wl.N, wl.eps)
    st = {}
    t = time.perf_counter()
    orc.binsort(X, prm.n, (16, 16, 8)[:wl.dim])
    st["sort"] = time.perf_counter() - t
    t = time.perf_counter()
    b = orc.spread(X, c, prm.n, prm.w, prm.beta)
    st["spread"] = time.perf_counter() - t
    t = time.perf_counter()
    orc.truncate_correct(orc.fft_forward(b), prm)
    st["fft1_deconv"] = time.perf_counter() - t
    t = time.perf_counter()
    g = orc.fft_backward(orc.precorrect_pad(f, prm))
    st["pad_fft2"] = time.perf_counter() - t
    t = time.perf_counter()
    orc.interp(X, g, prm.w, prm.beta)
    st["interp"] = time.perf_counter() - t
    return st


def cpu_baseline(wl, inp, sample_M):
    """The CPU oracle as it stands, on this host: all cores on the whole workload (its parallel
    spreading and interpolation, which equal the serial loops bit for bit, and a multi-threaded
    library FFT), and the plain serial oracle on the first `sample_M` points (one thread).  Both
    run the pair the benchmark times: bin-sort, type 1, type 2."""
    import oracle.oracle as orc
    orc._load()
    ncores = os.cpu_count() or 1
    try:
        ncores = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    threads = int(os.environ.get("OMP_NUM_THREADS", ncores))
    orc.THREADS, orc.FFT_WORKERS = threads, threads
    st_all = _oracle_pair(orc, wl, inp["X"], inp["c"], inp["f"])
    t_all = sum(st_all.values())
    orc.THREADS, orc.FFT_WORKERS = 1, 1
    X = [x[:sample_M] for x in inp["X"]]
    st_ser = _oracle_pair(orc, wl, X, inp["c"][:sample_M], inp["f"])
    t_ser = sum(st_ser.values())
    return {"value": wl.M / t_all, "unit": "NU points/s", "cores": threads, "kind": "oracle",
            "sample": f"all {wl.M} points of the same workload through the oracle on {threads} threads "
                      f"(bin-sort, type 1, type 2; parallel spread/interp, threaded scipy FFT), {t_all:.1f} s",
            "cpu_model": _cpu_model(), "nproc": ncores,
            "stages_s": {k: round(v, 3) for k, v in st_all.items()},
            "serial": {"value": sample_M / t_ser, "unit": "NU points/s", "cores": 1,
                       "sample": f"first {sample_M} of {wl.M} points, serial oracle, one-thread FFT, {t_ser:.1f} s",
                       "stages_s": {k: round(v, 3) for k, v in st_ser.items()}}}


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None when
    the kernel's source has changed since the counters were taken."""
    import glob
    import hashlib
    for path in glob.glob(os.path.join(ROOT, "profiles", "*hbm_traffic*.md")):
        for line in open(path):
            parts = line.split()
            if len(parts) < 2 or parts[0] != "traffic":
                continue
            kv = dict(p.split("=", 1) for p in parts[1:] if "=" in p)
            if kv.get("kernel") != kernel:
                continue
            src = os.path.join(ROOT, kv["source"])
            if not os.path.exists(src):
                return None
            if hashlib.sha256(open(src, "rb").read()).hexdigest() != kv.get("sha256"):
                return None
            return float(kv["bytes"])
    return None


def probe_copy(nbytes):
    """A plain device-to-device copy of known size, for calibrating the HBM byte counters."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    a.fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"probe_copy_bytes": nbytes, "copies": 3}))


def compare_methods(steps, workloads):
    """Method comparison (GM vs GM-sort vs SM, uniform vs clustered points): one JSON line per
    (workload, method, type) with NU points/s for exec (execute only, points already set), total
    (setpts + execute) and total+mem (host-to-device copies of the inputs from pinned memory,
    setpts, execute, and the copy of the output back)."""
    import numpy as np
    import torch

    import nonuniform_fft_amd as nf
    from nonuniform_fft_amd.workloads import WORKLOADS, make_inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    for name in workloads:
        wl = WORKLOADS[name]
        inp = make_inputs(wl)
        cdt = torch.complex64 if wl.precision == "f32" else torch.complex128
        hX = [torch.from_numpy(x).pin_memory() for x in inp["X"]]
        hc = torch.from_numpy(inp["c"]).pin_memory()
        hf = torch.from_numpy(inp["f"]).pin_memory()
        X = [x.to(dev) for x in hX]
        c_in = hc.to(dev)
        f_in = hf.to(dev)
        f_out = torch.empty(tuple(reversed(wl.N)), dtype=cdt, device=dev)
        c_out = torch.empty(wl.M, dtype=cdt, device=dev)
        hf_out = torch.empty(f_out.shape, dtype=cdt).pin_memory()
        hc_out = torch.empty(wl.M, dtype=cdt).pin_memory()
        for method, mname in ((2, "SM"), (1, "GM-sort"), (3, "GM")):
            for typ in (1, 2):
                plan = nf.Plan(typ, wl.N, wl.eps, wl.precision, stream=stream, method=method)

                def run_exec():
                    if typ == 1:
                        plan.execute(c_in, f_out)
                    else:
                        plan.execute(c_out, f_in)

                def run_total():
                    plan.setpts(*X)
                    run_exec()

                def run_mem():
                    for d, h in zip(X, hX):
                        d.copy_(h, non_blocking=True)
                    if typ == 1:
                        c_in.copy_(hc, non_blocking=True)
                    else:
                        f_in.copy_(hf, non_blocking=True)
                    run_total()
                    if typ == 1:
                        hf_out.copy_(f_out, non_blocking=True)
                    else:
                        hc_out.copy_(c_out, non_blocking=True)

                plan.setpts(*X)
                run_exec()
                res = {}
                for key, fn in (("exec", run_exec), ("total", run_total), ("total+mem", run_mem)):
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    for _ in range(steps):
                        fn()
                    torch.cuda.synchronize()
                    ms = (time.perf_counter() - t0) * 1e3 / steps
                    res[key] = {"ms": ms, "pts_per_s": wl.M / (ms * 1e-3)}
                plan.destroy()
                print(json.dumps({"workload": name, "method": mname, "type": typ, **res}), flush=True)


def many_vectors(steps, nvec, workloads):
    """Many-vector execution on one setpts: per workload, nvec type 1 + adjoint type 2 pairs as
    nvec single executes and as one execute_many + execute_adjoint_many; one JSON line each with
    the time per vector pair and NU points/s (points already set, inputs in HBM)."""
    import numpy as np
    import torch

    import nonuniform_fft_amd as nf
    from nonuniform_fft_amd.workloads import WORKLOADS, make_inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    for name in workloads:
        wl = WORKLOADS[name]
        X = [torch.from_numpy(x).to(dev) for x in make_inputs(wl, want_c=False, want_f=False)["X"]]
        rng = np.random.default_rng(5)
        cdt = torch.complex64 if wl.precision == "f32" else torch.complex128
        fshape = (nvec,) + tuple(reversed(wl.N))
        c_in = torch.complex(torch.from_numpy(rng.standard_normal((nvec, wl.M))),
                             torch.from_numpy(rng.standard_normal((nvec, wl.M)))).to(cdt).to(dev)
        f_in = torch.complex(torch.from_numpy(rng.standard_normal(fshape)),
                             torch.from_numpy(rng.standard_normal(fshape))).to(cdt).to(dev)
        f_out = torch.empty(fshape, dtype=cdt, device=dev)
        c_out = torch.empty((nvec, wl.M), dtype=cdt, device=dev)
        plan = nf.Plan(1, wl.N, wl.eps, wl.precision)
        plan.setpts(*X)

        def single():
            for v in range(nvec):
                plan.execute(c_in[v], f_out[v])
                plan.execute_adjoint(c_out[v], f_in[v])

        def many():
            plan.execute_many(c_in, f_out)
            plan.execute_adjoint_many(c_out, f_in)

        res = {}
        for key, fn in (("single", single), ("many", many)):
            fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / (steps * nvec)
            res[key] = {"ms_per_vector_pair": ms, "pts_per_s": wl.M / (ms * 1e-3)}
        plan.destroy()
        print(json.dumps({"workload": name, "nvec": nvec, **res}), flush=True)


def type3_bench(steps):
    """Type 3 timing: M sources uniform in [-pi, pi)^d, K targets uniform in [-F, F)^d (F = N/2,
    so the space-bandwidth product matches a type 1 of N^d modes); one JSON line per case with
    setpts and execute times and sources+targets per second of execute."""
    import numpy as np
    import torch

    import nonuniform_fft_amd as nf

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cases = [(3, 1 << 22, 1 << 22, 128, 1e-5, "f32"), (2, 1 << 22, 1 << 22, 1024, 1e-5, "f32"),
             (1, 1 << 24, 1 << 24, 1 << 20, 1e-6, "f32")]
    for d, M, K, N, eps, prec in cases:
        rng = np.random.default_rng(1010 + d)
        rd = np.float32 if prec == "f32" else np.float64
        X = [torch.from_numpy(rng.uniform(-np.pi, np.pi, M).astype(rd)).to(dev) for _ in range(d)]
        S = [torch.from_numpy(rng.uniform(-N / 2, N / 2, K).astype(rd)).to(dev) for _ in range(d)]
        cdt = torch.complex64 if prec == "f32" else torch.complex128
        c = torch.randn(M, dtype=cdt, device=dev)
        f = torch.empty(K, dtype=cdt, device=dev)
        p = nf.Plan(3, d, eps, prec)
        p.setpts_type3(X, S)
        p.execute(c, f)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            p.setpts_type3(X, S)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(steps):
            p.execute(c, f)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        set_ms, ex_ms = (t1 - t0) * 1e3 / steps, (t2 - t1) * 1e3 / steps
        print(json.dumps({"type3": f"{d}D M={M} K={K} targets in [-{N // 2}, {N // 2})^{d} {prec} eps={eps:g}",
                          "fine_grid": list(p.n), "setpts_ms": set_ms, "exec_ms": ex_ms,
                          "pts_per_s_exec": (M + K) / (ex_ms * 1e-3)}), flush=True)
        p.destroy()


def distribution_stress():
    """Stage times (HIP events, best of 3 after a warm-up) of the headline workload with its
    points drawn uniform, Gaussian-clustered and inside an 8-cell box, for SM and GM-sort; one
    JSON line per (distribution, method)."""
    import torch

    import nonuniform_fft_amd as nf
    from nonuniform_fft_amd.workloads import WORKLOADS, make_inputs, scaled

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    base = WORKLOADS["3d_n128_m16m_f32_e5"]
    for dist in ("uniform", "cluster", "box"):
        wl = base if dist == "uniform" else scaled(base, dist=dist)
        inp = make_inputs(wl)
        X = [torch.from_numpy(x).to(dev) for x in inp["X"]]
        c = torch.from_numpy(inp["c"]).to(dev)
        f = torch.from_numpy(inp["f"]).to(dev)
        fo = torch.empty(tuple(reversed(wl.N)), dtype=c.dtype, device=dev)
        co = torch.empty(wl.M, dtype=c.dtype, device=dev)
        for method in (2, 1):
            p = nf.Plan(1, wl.N, wl.eps, wl.precision, timing=True, method=method)
            res = {}
            for k in range(4):
                p.setpts(*X)
                p.execute(c, fo)
                p.execute_adjoint(co, f)
                torch.cuda.synchronize()
                st = p.stage_times()
                if k:
                    for key in ("sort", "spread", "interp"):
                        res[key] = min(res.get(key, 1e9), st[key])
            print(json.dumps({"dist": dist, "method": method, "nsub": p.info()["nsubproblems"],
                              **{k: round(v, 3) for k, v in res.items()}}), flush=True)
            p.destroy()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="3d_n128_m16m_f32_e5")
    ap.add_argument("--cpu-sample", type=int, default=1 << 22,
                    help="points of the workload timed on the CPU oracle (0 = skip)")
    ap.add_argument("--method", type=int, default=0)
    ap.add_argument("--upsampfac", type=float, default=0.0,
                    help="fine-grid upsampling factor sigma in [1.25, 2] (0 = 2)")
    ap.add_argument("--probe-copy", type=int, default=0,
                    help="only run a plain copy of this many bytes (counter calibration)")
    ap.add_argument("--compare", action="store_true",
                    help="only compare the GM, GM-sort and SM methods (JSON line per method and type)")
    ap.add_argument("--type3", action="store_true", help="only time type 3 transforms")
    ap.add_argument("--stress", action="store_true",
                    help="only time uniform / clustered / box point distributions (SM and GM-sort)")
    ap.add_argument("--many", type=int, default=0,
                    help="only time many-vector execution with this many vectors per call")
    args = ap.parse_args()
    if args.type3:
        type3_bench(args.steps)
        return
    if args.stress:
        distribution_stress()
        return
    if args.many:
        many_vectors(args.steps, args.many, ["2d_n64_m1e4_f32_e5", "2d_n1024_m4m_f32_e5", "3d_n128_m16m_f32_e5",
                                             "1d_n1m_m16m_f32_e6"])
        return
    if args.probe_copy:
        probe_copy(args.probe_copy)
        return
    if args.compare:
        compare_methods(args.steps, ["3d_n128_m16m_f32_e5", "3d_n128_m16m_f32_e5_cluster",
                                     "2d_n1024_m4m_f32_e5"])
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import nonuniform_fft_amd as nf
    from nonuniform_fft_amd.workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = make_inputs(wl)
    X = [torch.from_numpy(x).to(dev) for x in inp["X"]]
    c = torch.from_numpy(inp["c"]).to(dev)
    f_in = torch.from_numpy(inp["f"]).to(dev)
    cdt = torch.complex64 if wl.precision == "f32" else torch.complex128
    f_out = torch.empty(tuple(reversed(wl.N)), dtype=cdt, device=dev)
    c_out = torch.empty(wl.M, dtype=cdt, device=dev)
    stream = torch.cuda.current_stream()
    plan = nf.Plan(1, wl.N, wl.eps, wl.precision, stream=stream, timing=True, method=args.method,
                   upsampfac=args.upsampfac)

    def step():
        plan.setpts(*X)                   # bin-sort + subproblems
        plan.execute(c, f_out)            # type 1: spread, FFT, deconvolve
        plan.execute_adjoint(c_out, f_in)  # type 2 on the same sorted points

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    plan.stage_times()   # drops the warm-up steps' stage events

    keys = ["sort", "spread", "fft1", "deconv", "clear", "interp", "fft2", "pad"]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    # the plan's stage events of the timed steps (the last 16 at most), averaged; reading them
    # waits for the stream, which the closing synchronize does anyway
    st = plan.stage_times()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    stg = {k: st[k] for k in keys}

    rs = 4 if wl.precision == "f32" else 8
    info = plan.info()
    # dominant kernel: the spread (type 1 step 1) or the interpolation (type 2 step 3)
    bytes_alg = spread_bytes(wl.M, wl.dim, info["n"], rs)
    dom_name = "spread" if stg["spread"] >= stg["interp"] else "interp"
    dom_ms = stg[dom_name]
    achieved = bytes_alg / (dom_ms * 1e-3) / 1e9
    alu_tflops = wl.M * 4 * info["w"] ** wl.dim / (dom_ms * 1e-3) / 1e12
    exec1 = stg["clear"] + stg["spread"] + stg["fft1"] + stg["deconv"]
    exec2 = stg["pad"] + stg["fft2"] + stg["interp"]
    out = {
        "metric": "NU points/sec (type1 & type2, 3D fp32 eps=1e-5, spread+FFT+deconv) and % HBM roofline",
        "value": wl.M / (ms_step * 1e-3),
        "unit": "NU points/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.precision == "f32" else "f64",
        "data": "synthetic",
        "config": {"workload": f"{wl.dim}D type1+type2 pair N={'x'.join(map(str, wl.N))} M={wl.M} "
                               f"{wl.dist} {wl.precision} eps={wl.eps:g}"
                               + (f" sigma={args.upsampfac:g}" if args.upsampfac else ""),
                   "fine_grid": list(info["n"]), "w": info["w"], "bins": list(info["bins"]),
                   "nsubproblems": info["nsubproblems"]},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(dom_name) if args.workload == "3d_n128_m16m_f32_e5" else None,
                     "algorithmic_bytes": bytes_alg, "avg_ms": dom_ms},
        # the same kernel against the vector ALU: 4 flops per (point, cell) of complex x real
        # accumulate; peak = the published fp32 / fp64 vector rate (the fp32 figure counts packed
        # FMAs, which this build does not emit: its non-packed issue rate, 78.6 TFLOP/s, is given too)
        "roofline_alu": {"bound": "alu", "kernel": dom_name,
                         "achieved": alu_tflops,
                         "peak": 157.3 if wl.precision == "f32" else 78.6, "unit": "TFLOP/s",
                         "frac": alu_tflops / (157.3 if wl.precision == "f32" else 78.6),
                         "peak_nonpacked": 78.6, "frac_nonpacked": alu_tflops / 78.6},
        "stages_ms": stg,
        "exec_pts_per_s": {"type1": wl.M / (exec1 * 1e-3), "type2": wl.M / (exec2 * 1e-3)},
    }
    plan.destroy()
    if args.cpu_sample > 0:
        out["cpu_baseline"] = cpu_baseline(wl, inp, min(args.cpu_sample, wl.M))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
