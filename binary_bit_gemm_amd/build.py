"""Build liblowbit.so (HIP for gfx950) in-tree with hipcc.

    python -m binary_bit_gemm_amd.build [--jobs N] [--verbose] [--sanitize]

Every .hip / .cpp file under csrc/ is compiled to an object with hipcc for gfx950 and the
objects are linked into binary_bit_gemm_amd/liblowbit.so.  Packed FP32 instructions are
disabled for all device code.

--sanitize builds a separate, checking copy for CPU tests of the host code (argument checks,
planners, tile choice): binary_bit_gemm_amd/_build_san/liblowbit_san.so, with AddressSanitizer
and UndefinedBehaviorSanitizer on the host side only (the device code is built as usual).  A
process loads it with the sanitizer runtime preloaded (sanitizer_runtime() names it) and
LOWBIT_LIBRARY pointing at it.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblowbit.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # keep MFMA results in ordinary VGPRs: the per-group scale FMA reads every MFMA
          # result, and AGPR results would cost one v_accvgpr_read per element
          "-mllvm", "-amdgpu-mfma-vgpr-form=true",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


BUILD_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(BUILD_SAN, "liblowbit_san.so")
# host-side sanitizers only: every -fsanitize= stands right after -Xarch_host
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def sanitizer_runtime() -> str:
    """The shared AddressSanitizer runtime of the toolchain (preloaded by a process that loads the
    sanitized library; it carries the UndefinedBehaviorSanitizer handlers too)."""
    import glob as _g
    hits = sorted(_g.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang", "*", "lib",
                                       "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("no shared AddressSanitizer runtime found under the ROCm LLVM")
    return hits[-1]


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD_SAN if sanitize else BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + (SAN_HOST if sanitize else []) + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(jobs: int = 8, verbose: bool = False, sanitize: bool = False) -> str:
    os.makedirs(BUILD_SAN if sanitize else BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), srcs))
    lib = LIB_SAN if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if sanitize:  # link the shared sanitizer runtime (the loading process preloads it)
        rt = sanitizer_runtime()
        cmd += ["-L" + os.path.dirname(rt), "-Wl,-rpath," + os.path.dirname(rt), "-lclang_rt.asan-x86_64"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="build the host-sanitized copy for CPU tests (AddressSanitizer + UBSan, host code only)")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose, a.sanitize))


if __name__ == "__main__":
    main()
