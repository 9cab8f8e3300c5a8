"""Dropless mixture-of-experts layer hot path for AMD Instinct MI355X (gfx950).

The computation lives in the HIP library libmoe.so (C ABI in include/moe.h); this package
holds its ctypes binding (`_lib`, functions named like the C entry points) and the layer
composition (`layer`). Importing `_lib` fails loudly when the library is not built.
"""
from .build import build  # noqa: F401
