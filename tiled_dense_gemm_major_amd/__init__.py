"""libtgemm: block-tiled dense GEMM (fp16/bf16 in, fp32 sums, 16-bit out) for MI355X.

The product runs in hand-written gfx950 HIP kernels behind the C ABI of
``include/tgemm.h`` (``libtgemm.so``); ``tgemm`` is the ctypes binding.  Importing this
package loads nothing: the library is opened on first use and a missing library raises.
"""
from __future__ import annotations

_BINDING = ("gemm_f16", "gemm_bf16", "gemm_ex", "gemm_strided", "gemm", "query_config",
            "list_configs", "status_string", "version", "Config", "TGemmError", "F16", "BF16",
            "B_NK", "B_KN", "A_MK", "A_KM", "KERNEL_GENERIC", "KERNEL_TILED", "KERNEL_SKINNY", "KERNEL_DMA",
            "KERNEL_PINGPONG")


def __getattr__(name):
    if name in _BINDING:
        from . import tgemm
        return getattr(tgemm, name)
    raise AttributeError(name)
