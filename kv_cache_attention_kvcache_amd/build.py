"""Build libkvc.so (the HIP kernels and the C ABI) in-tree for gfx950.

Each ``csrc/*.hip`` file is compiled to an object under ``_build/`` (in
parallel), then they are linked into ``libkvc.so`` next to this file.  The
measured-ceiling kernels (``ceilings/*.hip``) go into their own
``ceilings/libkvc_ceilings.so``, so libkvc exports only the attention calls.
Each library is replaced atomically so a running process never loads a half
written file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libkvc.so")
CEIL_DIR = os.path.join(HERE, "ceilings")
CEIL_LIB_PATH = os.path.join(CEIL_DIR, "libkvc_ceilings.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvc)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(os.path.dirname(src)) + "_" + os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", os.path.dirname(src), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, path)


# The host side of the C entry points (argument validation, dispatch) under AddressSanitizer and
# UndefinedBehaviorSanitizer.  Only host code is instrumented: each -fsanitize= sits behind
# -Xarch_host, so the device code is the same as in libkvc.so.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_DIR = os.path.join(BUILD_DIR, "sanitize")
SAN_LIB_PATH = os.path.join(SAN_DIR, "libkvc.so")


def asan_runtime() -> str:
    """The ASan runtime of the ROCm compiler, which a process must preload to load the sanitized library."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("the ROCm compiler's ASan runtime is not installed")
    return found[-1]


def build_sanitized(verbose: bool = False) -> str:
    """libkvc.so with its host code under ASan + UBSan, in _build/sanitize/; returns its path."""
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc(), *FLAGS, *SANITIZE_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = SAN_LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE_FLAGS, "-shared-libsan", *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    os.replace(tmp, SAN_LIB_PATH)
    if verbose:
        print(f"built {SAN_LIB_PATH}")
    return SAN_LIB_PATH


def build(verbose: bool = False) -> str:
    """Compile every kernel source, link libkvc.so and libkvc_ceilings.so; returns libkvc's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    ceil_srcs = sorted(glob.glob(os.path.join(CEIL_DIR, "*.hip")))
    if not srcs or not ceil_srcs:
        raise RuntimeError("no HIP sources found")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(ceil_srcs))) as ex:
        objs = list(ex.map(_compile, srcs + ceil_srcs))
    _link(objs[:len(srcs)], LIB_PATH)
    _link(objs[len(srcs):], CEIL_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources and {CEIL_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
