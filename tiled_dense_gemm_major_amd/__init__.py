"""libtgemm: block-tiled dense GEMM (fp16/bf16 in, fp32 sums, 16-bit out) for MI355X.

The product runs in hand-written gfx950 HIP kernels behind the C ABI of
``include/tgemm.h`` (``libtgemm.so``); ``tgemm`` is the ctypes binding, and every public
name of it (``tgemm.__all__``) is also reachable here.  Importing this package loads
nothing: the library is opened on first use and a missing library raises.
"""
from __future__ import annotations

import importlib


def _binding():
    return importlib.import_module(__name__ + ".tgemm")


def __getattr__(name):
    if name.startswith("__"):
        raise AttributeError(name)
    b = _binding()
    if name in b.__all__:
        return getattr(b, name)
    raise AttributeError(name)


def __dir__():
    return sorted(set(globals()) | set(_binding().__all__))
