"""Builds libcb.so in-tree with hipcc for gfx950 (runs here without a GPU).

    python -m ragged_continuous_batching_amd.build [-j N] [--sanitize]

Every HIP translation unit is compiled with packed-fp32 instruction selection disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the hand-written kernels use no
packed fp32 arithmetic either. Host-only sources (``*.cpp``) are compiled as C++.

``--device-checks`` builds a debug copy, ``_build/checks/libcb.so``, whose kernels also count
every block id outside the pool that they meet (they read block 0 in its place, as every
build does); ``cb_debug_violations`` returns the count (tests/test_gpu_device_checks.py).

``--sanitize`` builds a test copy, ``_build/asan/libcb.so``, whose host code (the step
builder, the planner, argument checks, the entry points) carries AddressSanitizer and
UndefinedBehaviorSanitizer checks; device code is built as usual (each ``-fsanitize=``
follows ``-Xarch_host``). A process loads it with the clang ASan runtime preloaded and
``CB_LIBRARY`` pointing at it (tests/test_sanitized_host.py).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcb.so")
ASAN_BUILD = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_BUILD, "libcb.so")
CHECKS_BUILD = os.path.join(BUILD, "checks")
CHECKS_LIB = os.path.join(CHECKS_BUILD, "libcb.so")
# host-side sanitizers; every flag behind -Xarch_host so device code is not instrumented
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-shared-libasan", "-g"]
ARCH = "gfx950"


def hipcc() -> str:
    return os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def common_flags():
    return ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def compile_one(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-x", "hip", "-c", src, "-o", obj,
               *common_flags(),
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *extra]
    else:
        rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
        cmd = [hipcc(), "-x", "c++", "-c", src, "-o", obj, *common_flags(), f"-I{rocm}/include",
               "-D__HIP_PLATFORM_AMD__=1", *extra]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False, sanitize: bool = False, device_checks: bool = False) -> str:
    if sanitize:
        out_dir, lib, extra = ASAN_BUILD, ASAN_LIB, SANITIZE
    elif device_checks:
        out_dir, lib, extra = CHECKS_BUILD, CHECKS_LIB, ["-DCB_DEVICE_CHECKS"]
    else:
        out_dir, lib, extra = BUILD, LIB, []
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda src: compile_one(src, out_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs, *extra]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that a sanitized build links against."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
        found = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                              "libclang_rt.asan-x86_64.so")))
        if not found:
            raise RuntimeError("clang ASan runtime not found")
        path = found[-1]
    return path


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--sanitize", action="store_true", help="the host-sanitized test copy in _build/asan")
    ap.add_argument("--device-checks", action="store_true", help="the debug copy with device checks in _build/checks")
    args = ap.parse_args(argv)
    build(args.j, verbose=True, sanitize=args.sanitize, device_checks=args.device_checks)


if __name__ == "__main__":
    sys.exit(main())
