"""Build a host-sanitized copy of the library for CPU-only test runs.

    python -m image_generation_qi_amd.build_sanitized

Every source is compiled as in build.py, with AddressSanitizer and UndefinedBehaviorSanitizer
applied to the host code only (each sanitizer flag follows -Xarch_host, so the gfx950 device
code is built exactly as in the product library), and linked by the ROCm clang++ against its
shared sanitizer runtime into image_generation_qi_amd/libqi_san.so.  That file is for CPU runs of
the host tests (layout analysis, tables, block maps, workspace sizes and every argument check
before a launch); it is never loaded on a GPU.  Run it with the sanitizer runtime preloaded, as
tests/test_host_sanitized.py does (sanitizer_env gives the environment).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

from . import build as B

BUILD_SAN = os.path.join(B.PKG, "_build_san")
LIB_SAN = os.path.join(B.PKG, "libqi_san.so")
HOST_SAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def llvm_bin(name: str) -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(root, "lib", "llvm", "bin", name)


def asan_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the ROCm clang (preloaded for test runs)."""
    r = subprocess.run([llvm_bin("clang++"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"sanitizer runtime not found ({path!r})")
    return path


def sanitizer_env(base=None) -> dict:
    """Environment for a CPU process that loads libqi_san.so: the runtime preloaded, leaks not
    reported (the interpreter keeps its allocations at exit), the first error fatal."""
    env = dict(os.environ if base is None else base)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = asan_runtime() + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:detect_odr_violation=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["QI_LIBRARY"] = LIB_SAN
    return env


def compile_one(src: str) -> str:
    obj = os.path.join(BUILD_SAN, os.path.basename(src) + ".o")
    cmd = [B.hipcc()] + [f for f in B.common_flags() if f != "-O3"] + HOST_SAN_FLAGS
    if src.endswith(".hip"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(B.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    return obj


def build_sanitized(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD_SAN, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = LIB_SAN + ".tmp"
    # host link only: the objects already carry their gfx950 code objects
    cmd = [llvm_bin("clang++"), "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan", "-o", tmp] + \
        objs + ["-L", os.path.join(rocm, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_SAN)
    if verbose:
        print(f"built {LIB_SAN}")
    return LIB_SAN


if __name__ == "__main__":
    build_sanitized(jobs=min(8, os.cpu_count() or 4), verbose=True)
    sys.exit(0)
