"""Build libdflash.so (gfx950) in-tree with hipcc.

    python block_diffusion_drafter_rmsnorm_amd/build.py     (or __graft_entry__.build())

Each translation unit compiles in its own hipcc process (in parallel), then
one link step writes block_diffusion_drafter_rmsnorm_amd/libdflash.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libdflash.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"
SOURCES = ["gemm.hip", "attention.hip", "misc.hip", "sampling.hip", "selector.hip", "reserve.hip",
           "noalloc.hip", "check.hip", "api.cpp"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 vector ops stay off (plain scalar fp32 code only)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the C ABI layer
# (argument checks, workspace layout, scratch lookup); the kernels are the
# regular objects.  Each -fsanitize= applies to the host compilation only.
SAN_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-I", os.path.join(ROOT, "include")]
SAN_SOURCES = ["api.cpp", "noalloc.hip"]
SAN_OUT = os.path.join(BUILD, "libdflash_sanitized.so")


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime the sanitized library links against."""
    r = subprocess.run([os.path.join(os.path.dirname(hipcc()), "..", "lib", "llvm", "bin",
                        "clang++"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return path


def build_sanitized(verbose: bool = True) -> str:
    """_build/libdflash_sanitized.so (for the CPU tests of the C ABI)."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src in SAN_SOURCES:
            obj = os.path.join(BUILD, src + ".san.o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [hipcc(), *SAN_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
        else:
            obj = os.path.join(BUILD, os.path.basename(src) + ".o")
            if not os.path.exists(obj):
                obj = _compile(src)
        objs.append(obj)
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *objs,
           "-o", SAN_OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "sanitized":
        build_sanitized()
    else:
        build()
    sys.exit(0)
