"""Host AddressSanitizer build of the library: the host code (the C entry points, their
argument checks, workspace arithmetic and launch set-up) instrumented with ASan, the device
code as in the release build. For CPU runs of the host-side tests only; never loaded on a
GPU. The process must preload the ASan runtime (runtime() gives its path) and set MOE_LIB to
the library this builds."""
from __future__ import annotations

import glob
import os

from .build import BUILD, HIPCC, build_variant

ASAN_LIB = os.path.join(BUILD, "asan", "libmoe_asan.so")
# the sanitizer applies to the host pass only (each flag behind -Xarch_host)
ASAN_COMPILE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-O1"]
ASAN_LINK = ["-Xarch_host", "-fsanitize=address", "-shared-libsan"]


def runtime() -> str | None:
    """The clang ASan runtime that matches hipcc's host compiler, or None."""
    root = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    hits = sorted(glob.glob(os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")) +
                  glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build() -> str:
    return build_variant(ASAN_LIB, os.path.join(BUILD, "asan"), ASAN_COMPILE, ASAN_LINK)


if __name__ == "__main__":
    print(build())
