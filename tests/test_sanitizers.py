"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code,
run on the CPU (no GPU needed).

* The oracle (oracle/mx_oracle.c) built with gcc under both sanitizers, and
  its pins (tests/test_oracle_*.py) run on that build.
* The library's host code -- argument validation, workspace sizing, launch
  planning and dispatch in csrc/mx_api.cpp and csrc/mx_plan.cpp -- built
  with g++ under both sanitizers against tests/sanitize/host_stubs.cpp (a
  fake gfx950 device and counting kernel launchers), and driven through every
  entry point by tests/sanitize/host_checks.py.
Any sanitizer finding aborts the child process and fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "microscaling_quantized_linear_amd", "csrc")


def _asan_runtime():
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc / g++ not found")
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("no AddressSanitizer runtime")
    return path


def _env(asan, **extra):
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4", **extra)
    return env


def _host_lib(tmp_path):
    lib = str(tmp_path / "libmx_host_san.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", os.path.join(CSRC, "mx_api.cpp"),
           os.path.join(CSRC, "mx_plan.cpp"), os.path.join(ROOT, "tests", "sanitize",
                                                           "host_stubs.cpp"), "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "hip_runtime.h" in r.stderr:
        pytest.skip("HIP headers not found")
    assert r.returncode == 0, r.stderr[-3000:]
    return lib


def test_host_code_under_sanitizers(tmp_path):
    asan = _asan_runtime()
    lib = _host_lib(tmp_path)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "host_checks.py"),
                        lib], capture_output=True, text=True, env=_env(asan), timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host checks ok" in r.stdout
    assert "mx: " not in r.stderr, "dispatch trace printed without MX_LOG"


def test_dispatch_trace(tmp_path):
    """MX_LOG=1: one stderr line per launch decision, naming the kernel and its
    plan, for every family of the hot path (run on the sanitized host build,
    whose fake gfx950 device lets every dispatch through to counting stubs)."""
    asan = _asan_runtime()
    lib = _host_lib(tmp_path)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "host_checks.py"),
                        lib], capture_output=True, text=True, env=_env(asan, MX_LOG="1"),
                       timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("mx: ")]
    for kernel in ("gemv_w8_fused_kernel", "gemm_w8a8_kernel", "quant_act_t16_kernel",
                   "gemv_kernel", "moe_combine_kernel"):
        assert any(kernel in ln for ln in lines), f"no trace line for {kernel}"
    assert all("M=" in ln or "T=" in ln for ln in lines)


def test_oracle_pins_under_sanitizers(tmp_path):
    asan = _asan_runtime()
    sys.path.insert(0, ROOT)
    import oracle
    lib = oracle.build(str(tmp_path / "libmx_oracle_san.so"), sanitize=True)
    pins = sorted(os.path.join(ROOT, "tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                  if f.startswith("test_oracle_") and f.endswith(".py"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *pins],
                       capture_output=True, text=True, env=_env(asan, MX_ORACLE_LIB=lib),
                       timeout=900, cwd=str(tmp_path))
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout
