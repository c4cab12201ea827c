"""Build libgptq.so (gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, then linked into ``_lib/libgptq.so`` next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "libgptq.so")

SOURCES = ["panel_row_group.hip", "panel_row_grid.hip", "abi.cpp", "hessian.hip", "factor.hip", "gemm.hip",
           "quantize.hip", "packed.hip", "gptq2d.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", "-Wno-unused-variable",
         f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
LIB_SAN = os.path.join(BUILD, "libgptq_sanitized.so")


def build_sanitized(verbose: bool = False) -> str:
    """libgptq with the C ABI layer (abi.cpp: argument validation, planning calls,
    dispatch) built with AddressSanitizer and UndefinedBehaviorSanitizer on the
    host side, linked with the kernels' objects of the normal build.  Loaded with
    the sanitizer runtime preloaded (the CPU ABI tests run that way); never used
    on a GPU.  Rebuilt when abi.cpp, the headers or the objects are newer."""
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "abi.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    deps = [os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "gptq_internal.h"),
            os.path.join(INCLUDE, "gptq.h"), *objs]
    if os.path.exists(LIB_SAN) and os.path.getmtime(LIB_SAN) >= max(os.path.getmtime(d) for d in deps):
        return LIB_SAN
    abi = os.path.join(BUILD, "abi_sanitized.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"]
    for cmd in ([hipcc(), "-x", "hip", *flags, *SANITIZE, "-c", os.path.join(CSRC, "abi.cpp"), "-o", abi],
                [hipcc(), "-shared", f"--offload-arch={ARCH}", *SANITIZE, "-o", LIB_SAN + ".tmp", abi, *objs]):
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"sanitized build failed:\n{res.stdout}{res.stderr}")
    os.replace(LIB_SAN + ".tmp", LIB_SAN)
    return LIB_SAN


def sanitizer_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to preload)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang"
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True, check=True)
    return res.stdout.strip()


if __name__ == "__main__":
    build()
