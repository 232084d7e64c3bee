"""Compile liblora.so (HIP, gfx950) in-tree with hipcc.

    python -m lora_adapter_amd.build              # build
    python -m lora_adapter_amd.build --clean      # remove objects first
    python -m lora_adapter_amd.build --sanitize   # host code under ASan + UBSan

Objects go to lora_adapter_amd/_build/, the library to lora_adapter_amd/liblora.so.
The sanitized build (host code only instrumented, device code as usual, at -O1)
goes to lora_adapter_amd/_build_san/liblora_san.so; it needs the clang address
sanitizer runtime preloaded (asan_runtime()).
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
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblora.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblora)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off: the compiler must not emit v_pk_*_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


SAN_DIR = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(SAN_DIR, "liblora_san.so")
# each sanitizer flag right after -Xarch_host: instrument the host code only
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The clang address sanitizer runtime that the sanitized library needs
    preloaded into the host process ('' if this toolchain has none)."""
    pat = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm", "lib", "clang",
                       "*", "lib", "linux", "libclang_rt.asan-x86_64.so")
    found = sorted(glob.glob(pat)) or sorted(glob.glob(
        "/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else ""


def _compile_san(src: str) -> str:
    obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *[f for f in COMMON if f != "-O3"], "-O1", "-g", *SAN_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build_sanitized(verbose: bool = False) -> str:
    """The library with its host code under the address and undefined-behaviour
    sanitizers (for the CPU tests of the C ABI and the host page table)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(6, len(srcs))) as ex:
        objs = list(ex.map(_compile_san, srcs))
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS[:2], *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def build(clean: bool = False, verbose: bool = False) -> str:
    if clean and os.path.isdir(OBJDIR):
        shutil.rmtree(OBJDIR)
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(6, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--clean", action="store_true")
    ap.add_argument("--sanitize", action="store_true")
    args = ap.parse_args()
    if args.sanitize:
        build_sanitized(verbose=True)
    else:
        build(clean=args.clean, verbose=True)
    sys.exit(0)
