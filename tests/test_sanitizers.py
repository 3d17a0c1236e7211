"""Sanitizer runs on the CPU: the oracle's C routines built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, host code only) and driven by tests/oracle_sanitize_driver.c,
which calls every routine on small, folded, wrapped, empty and rejected inputs."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "nufft_oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="3")
    r = subprocess.run([str(exe)], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_abi_host_checks_under_asan_ubsan(tmp_path):
    """The C ABI's host-side argument checks with plan.cpp built under AddressSanitizer and
    UndefinedBehaviorSanitizer (host code only: -Xarch_host), linked with the library's other
    objects from the regular build; leak detection on."""
    hipcc = "/opt/rocm/bin/hipcc"
    clangxx = "/opt/rocm/lib/llvm/bin/clang++"
    objdir = os.path.join(ROOT, "nonuniform_fft_amd", "_build")
    others = [os.path.join(objdir, f"{s}.o") for s in ("binsort", "spread", "interp", "deconv", "t3")]
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)) or not all(os.path.exists(o) for o in others):
        pytest.skip("needs hipcc and the library's objects (run the build first)")
    inc = os.path.join(ROOT, "include")
    plan_o, drv_o, exe = tmp_path / "plan.o", tmp_path / "driver.o", tmp_path / "abi_sanitize"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    subprocess.run([hipcc, "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", inc, *san,
                    "-c", os.path.join(ROOT, "nonuniform_fft_amd", "csrc", "plan.cpp"), "-o", str(plan_o)],
                   check=True, capture_output=True, text=True)
    subprocess.run([clangxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", inc, "-c", os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp"), "-o", str(drv_o)],
                   check=True, capture_output=True, text=True)
    subprocess.run([hipcc, "--hip-link", "--offload-arch=gfx950", "-fsanitize=address,undefined", str(drv_o),
                    str(plan_o), *others, "-L/opt/rocm/lib", "-lrocfft", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe)], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
