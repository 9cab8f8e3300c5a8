"""Build libmoe.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build_variant(lib: str, out_dir: str, compile_extra=(), link_extra=()) -> str:
    """Compile every csrc/*.hip with the extra flags into out_dir and link `lib`."""
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, compile_extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


DEBUG_LIB = os.path.join(PKG, "libmoe_debug.so")


def build(verbose: bool = False, variant: str = "release") -> str:
    """Compile every csrc/*.hip and link libmoe.so next to this file. Always rebuilds.

    variant "debug": the same sources with MOE_DEBUG=1, linked as libmoe_debug.so next to it
    (the operand loads of the grouped GEMM range-checked by the hardware, the device index
    data validated on the host before each launch); load it by setting MOE_LIB to its path."""
    if variant == "debug":
        lib = build_variant(DEBUG_LIB, os.path.join(BUILD, "debug"), ["-DMOE_DEBUG=1"])
    elif variant == "release":
        lib = build_variant(LIB, BUILD)
    else:
        raise ValueError(variant)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
