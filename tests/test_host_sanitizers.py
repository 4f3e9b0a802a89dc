"""The host code of the library (argument checks, the kernel choice, the split-K and grouped
planners, the entry points' early returns) under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  The library is rebuilt with both sanitizers on its host side (device code as usual;
binary_bit_gemm_amd/build.py --sanitize), and the CPU ABI and planner tests run against that copy
in a child process with the sanitizer runtime preloaded; any report fails the run."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(lib: str) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = glob.glob(os.path.join(ROOT, "binary_bit_gemm_amd", "csrc", "*")) + [os.path.join(ROOT, "include", "lowbit.h")]
    return any(os.path.getmtime(s) > t for s in srcs)


def test_host_code_under_asan_and_ubsan():
    from binary_bit_gemm_amd import build as B
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc is not installed")
    rt = B.sanitizer_runtime()
    lib = B.LIB_SAN
    if _stale(lib):
        B.build(jobs=min(8, os.cpu_count() or 1), sanitize=True)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "LOWBIT_LIBRARY": lib,
        # Python's own allocations are not the subject: no leak report; stop at the first error
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=97",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=98",
    })
    env.pop("LOWBIT_VARIANT", None)
    env.pop("LOWBIT_RESIDENT_PLAN", None)
    # the child loads the sanitized copy with the runtime mapped
    probe = ("import binary_bit_gemm_amd as lb; lb.lib(); print(lb.library_path()); "
             "print(any('libclang_rt.asan' in l for l in open('/proc/self/maps')))")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.split() == [lib, "True"], r.stdout + r.stderr
    # the runtime is armed: a batched size query handed a problem array that ends 8 bytes short
    # (malloc'd, so the sanitizer's redzone follows it) reads past its end and must be reported
    canary = ("import ctypes, binary_bit_gemm_amd as lb; libc = ctypes.CDLL(None); "
              "libc.malloc.restype = ctypes.c_void_p; libc.malloc.argtypes = [ctypes.c_size_t]; "
              "n = ctypes.sizeof(lb.Problem) - 8; p = libc.malloc(n); "
              "ctypes.memmove(p, ctypes.byref(lb.Problem(256, 256, 256, 256, 16, 256, 6144, 64, 2)), n); "
              "lb.lib().lowbit_batched_workspace_size(ctypes.c_void_p(p), 1)")
    r = subprocess.run([sys.executable, "-c", canary], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, (r.returncode, r.stderr[-2000:])
    # the CPU tests of the host code, against the sanitized copy
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_host_planners.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, f"sanitized run failed (rc {r.returncode}):\n{out[-4000:]}"
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
