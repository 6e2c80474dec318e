"""Thin ctypes binding of libtgemm (include/tgemm.h): argument marshalling only.

Every step of the product runs in the library's HIP kernels; PyTorch, when used, only
supplies device memory (``data_ptr()``) and streams (``cuda_stream``).  There is no CPU
fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

F16, BF16 = 0, 1
B_NK, B_KN = 0, 1
A_MK, A_KM = 0, 1
(KERNEL_GENERIC, KERNEL_TILED, KERNEL_SKINNY, KERNEL_DMA, KERNEL_PINGPONG, KERNEL_QUAD,
 KERNEL_SPLITK, KERNEL_DIRECT, KERNEL_QUAD_SPLITK, KERNEL_QUAD_STREAMK,
 KERNEL_MASKED) = range(11)
# the kernels that take operands of any 2-byte alignment
ANY_ALIGNMENT_KERNELS = (KERNEL_GENERIC, KERNEL_MASKED)
SPLIT_KERNELS = (KERNEL_SPLITK, KERNEL_QUAD_SPLITK)   # split K over workgroups (workspace)
WORKSPACE_KERNELS = SPLIT_KERNELS + (KERNEL_QUAD_STREAMK,)   # need a lent workspace
STREAMK_WORKSPACE_BYTES = 128 << 20                   # a QUAD_STREAMK configuration's

SCRATCH_BYTES = 16 << 20    # the fixed per-GPU scratch of gemm_ex_noalloc
CLOCK_STAMP_SLOTS = 4096    # compute-unit slots of one clock stamp (2 int64 each)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtgemm.so")

EXPORTS = ("attn_fwd_f16", "gemm_f16", "gemm_bf16", "gemm_ex", "gemm_ex_ws", "gemm_ex_noalloc",
           "gemm_strided",
           "tgemm_query_config", "tgemm_query_config_ex", "tgemm_query_config_ws",
           "tgemm_workspace_size", "tgemm_list_configs", "tgemm_list_configs_ex",
           "tgemm_status_string", "tgemm_version", "tgemm_clock_stamp",
           "tgemm_wall_clock_hz")


__all__ = ["F16", "BF16", "B_NK", "B_KN", "A_MK", "A_KM", "KERNEL_GENERIC", "KERNEL_TILED",
           "KERNEL_SKINNY", "KERNEL_DMA", "KERNEL_PINGPONG", "KERNEL_QUAD", "KERNEL_SPLITK",
           "KERNEL_QUAD_SPLITK", "KERNEL_QUAD_STREAMK", "KERNEL_MASKED", "SPLIT_KERNELS",
           "WORKSPACE_KERNELS", "ALIGN_OPERANDS",
           "ANY_ALIGNMENT_KERNELS",
           "STREAMK_WORKSPACE_BYTES",
           "KERNEL_DIRECT",
           "LIB_PATH", "EXPORTS", "TGemmError", "Config", "load", "status_string", "gemm_f16",
           "gemm_bf16", "gemm_ex", "gemm_ex_ws", "gemm_ex_noalloc", "gemm_strided",
           "query_config", "SCRATCH_BYTES", "CLOCK_STAMP_SLOTS",
           "query_config_packed", "query_config_ws", "workspace_size", "list_configs",
           "attn_fwd_f16", "version", "gemm", "clock_stamp", "wall_clock_hz"]


class TGemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class Config(ctypes.Structure):
    """tgemm_config."""
    _fields_ = [("kernel", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("block_n", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("waves_m", ctypes.c_int32), ("waves_n", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("group_m", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("mfma", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}

    @classmethod
    def from_dict(cls, d: dict) -> "Config":
        return cls(**{name: int(d[name]) for name, _ in cls._fields_})

    def __repr__(self):
        return f"Config({self.as_dict()})"


_lib = None


def load(path: str = LIB_PATH):
    """Load libtgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it first (python -m tiled_dense_gemm_major_amd.build)")
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    cfgp = ctypes.POINTER(Config)
    lib.gemm_f16.argtypes = [i64, i64, i64, vp, vp, vp, i32, vp]
    lib.gemm_bf16.argtypes = [i64, i64, i64, vp, vp, vp, i32, vp]
    lib.gemm_ex.argtypes = [i32, i64, i64, i64, vp, vp, vp, i32, cfgp, vp]
    lib.gemm_ex_ws.argtypes = [i32, i64, i64, i64, vp, vp, vp, i32, cfgp, vp, i64, vp]
    lib.gemm_ex_noalloc.argtypes = [i32, i64, i64, i64, vp, vp, vp, i32, cfgp, vp]
    lib.attn_fwd_f16.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, i32, vp]
    lib.gemm_strided.argtypes = [i32, i64, i64, i64, vp, i64, i32, vp, i64, i32, vp, i64,
                                 cfgp, vp]
    lib.tgemm_query_config.argtypes = [i32, i64, i64, i64, i32, cfgp]
    lib.tgemm_query_config_ex.argtypes = [i32, i64, i64, i64, i32, i32, i32, cfgp]
    lib.tgemm_query_config_ws.argtypes = [i32, i64, i64, i64, i32, i32, cfgp,
                                          ctypes.POINTER(ctypes.c_int64)]
    lib.tgemm_workspace_size.argtypes = [i64, i64, cfgp, ctypes.POINTER(ctypes.c_int64)]
    lib.tgemm_list_configs.argtypes = [i32, i32, cfgp, i32]
    lib.tgemm_list_configs_ex.argtypes = [i32, i32, i32, cfgp, i32]
    lib.tgemm_clock_stamp.argtypes = [vp, vp]
    lib.tgemm_wall_clock_hz.argtypes = [ctypes.POINTER(ctypes.c_int64)]
    lib.tgemm_status_string.argtypes = [i32]
    lib.tgemm_status_string.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name != "tgemm_status_string":
            getattr(lib, name).restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().tgemm_status_string(status).decode()


def _addr(x) -> int:
    """A device address from a torch tensor, an int, or None (NULL)."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return int(torch.cuda.current_stream().cuda_stream)
        except ImportError:
            pass
        return 0
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(rc: int, what: str):
    if rc != 0:
        raise TGemmError(rc, what)


def gemm_f16(m, n, k, A, B, C, b_layout=B_NK, stream=None):
    """C = A x B^T (B_NK) or A x B (B_KN), fp16.  A, B, C: device tensors or addresses."""
    _check(load().gemm_f16(m, n, k, _addr(A), _addr(B), _addr(C), b_layout, _stream(stream)),
           "gemm_f16")


def gemm_bf16(m, n, k, A, B, C, b_layout=B_NK, stream=None):
    """C = A x B^T (B_NK) or A x B (B_KN), bf16.  A, B, C: device tensors or addresses."""
    _check(load().gemm_bf16(m, n, k, _addr(A), _addr(B), _addr(C), b_layout, _stream(stream)),
           "gemm_bf16")


def gemm_ex(dtype, m, n, k, A, B, C, b_layout=B_NK, config: Config | None = None,
            stream=None):
    """The product with an explicit dtype and, optionally, an explicit configuration."""
    cfg = ctypes.byref(config) if config is not None else None
    _check(load().gemm_ex(dtype, m, n, k, _addr(A), _addr(B), _addr(C), b_layout, cfg,
                          _stream(stream)), "gemm_ex")


def gemm_ex_ws(dtype, m, n, k, A, B, C, workspace, workspace_bytes, b_layout=B_NK,
               config: Config | None = None, stream=None):
    """gemm_ex with a caller-lent device workspace (split-K configurations need one)."""
    cfg = ctypes.byref(config) if config is not None else None
    _check(load().gemm_ex_ws(dtype, m, n, k, _addr(A), _addr(B), _addr(C), b_layout, cfg,
                             _addr(workspace) if workspace is not None else None,
                             int(workspace_bytes), _stream(stream)), "gemm_ex_ws")


def gemm_ex_noalloc(dtype, m, n, k, A, B, C, b_layout=B_NK, config: Config | None = None,
                    stream=None):
    """gemm_ex_ws with the library's fixed scratch as the workspace: allocates nothing."""
    cfg = ctypes.byref(config) if config is not None else None
    _check(load().gemm_ex_noalloc(dtype, m, n, k, _addr(A), _addr(B), _addr(C), b_layout, cfg,
                                  _stream(stream)), "gemm_ex_noalloc")


ALIGN_OPERANDS = 2   # `aligned` value: A and B meet the fast rules, C or N does not


def _align_arg(aligned) -> int:
    return ALIGN_OPERANDS if (not isinstance(aligned, bool) and aligned == ALIGN_OPERANDS) \
        else int(bool(aligned))


def query_config_ws(dtype, m, n, k, b_layout=B_NK, aligned=True):
    """(configuration, workspace bytes) the table picks when a workspace can be lent;
    aligned: True (every fast-kernel rule), False (none) or ALIGN_OPERANDS."""
    out = Config()
    nbytes = ctypes.c_int64(0)
    _check(load().tgemm_query_config_ws(dtype, m, n, k, b_layout, _align_arg(aligned),
                                        ctypes.byref(out), ctypes.byref(nbytes)),
           "tgemm_query_config_ws")
    return out, int(nbytes.value)


def workspace_size(m, n, config: Config) -> int:
    nbytes = ctypes.c_int64(0)
    _check(load().tgemm_workspace_size(m, n, ctypes.byref(config), ctypes.byref(nbytes)),
           "tgemm_workspace_size")
    return int(nbytes.value)


def gemm_strided(dtype, m, n, k, A, lda, a_layout, B, ldb, b_layout, C, ldc,
                 config: Config | None = None, stream=None):
    """The general product: A [M,K] (A_MK) or [K,M] (A_KM), B [N,K] (B_NK) or [K,N] (B_KN),
    C [M,N], each with a leading dimension in elements."""
    cfg = ctypes.byref(config) if config is not None else None
    _check(load().gemm_strided(dtype, m, n, k, _addr(A), lda, a_layout, _addr(B), ldb,
                               b_layout, _addr(C), ldc, cfg, _stream(stream)), "gemm_strided")


def query_config(dtype, m, n, k, b_layout=B_NK, aligned=True, a_layout=A_MK) -> Config:
    """The choice for an alignment class: aligned True (every fast-kernel rule), False
    (none: the masked kernel) or ALIGN_OPERANDS (A and B meet the rules, C or N does not)."""
    out = Config()
    _check(load().tgemm_query_config_ex(dtype, m, n, k, a_layout, b_layout,
                                        _align_arg(aligned), ctypes.byref(out)),
           "tgemm_query_config_ex")
    return out


def query_config_packed(dtype, m, n, k, b_layout=B_NK) -> Config:
    """What gemm_f16 / gemm_bf16 pick for packed operands at 16-byte-aligned addresses
    (tgemm_query_config: the sizes decide whether the fast kernels apply)."""
    out = Config()
    _check(load().tgemm_query_config(dtype, m, n, k, b_layout, ctypes.byref(out)),
           "tgemm_query_config")
    return out


def list_configs(dtype, b_layout=B_NK, a_layout=A_MK) -> list:
    lib = load()
    count = lib.tgemm_list_configs_ex(dtype, a_layout, b_layout, None, 0)
    if count < 0:
        raise TGemmError(count, "tgemm_list_configs_ex")
    arr = (Config * count)()
    lib.tgemm_list_configs_ex(dtype, a_layout, b_layout, arr, count)
    return [arr[i] for i in range(count)]


def attn_fwd_f16(batch, seq, heads, dim, Q, K, V, O, causal=True, stream=None):
    """Attention forward, fp16 tensors [batch, seq, heads, dim]: O = softmax(Q K^T /
    sqrt(dim)) V per (batch, head), causal or not.  Q, K, V, O: device tensors or
    addresses."""
    _check(load().attn_fwd_f16(batch, seq, heads, dim, _addr(Q), _addr(K), _addr(V), _addr(O),
                               int(bool(causal)), _stream(stream)), "attn_fwd_f16")


def clock_stamp(out, stream=None):
    """Enqueue per-compute-unit (engine-clock counter, wall clock) stamps into ``out`` (a
    zeroed device tensor of CLOCK_STAMP_SLOTS x 2 int64, 16-byte aligned, or an
    address)."""
    if hasattr(out, "numel") and out.numel() < 2 * CLOCK_STAMP_SLOTS:
        raise ValueError(f"clock_stamp needs {2 * CLOCK_STAMP_SLOTS} int64, got {out.numel()}")
    _check(load().tgemm_clock_stamp(_addr(out), _stream(stream)), "tgemm_clock_stamp")


def wall_clock_hz() -> int:
    hz = ctypes.c_int64(0)
    _check(load().tgemm_wall_clock_hz(ctypes.byref(hz)), "tgemm_wall_clock_hz")
    return int(hz.value)


def version() -> int:
    return int(load().tgemm_version())


def gemm(A, B, C=None, b_layout=B_NK, config: Config | None = None, stream=None):
    """Torch convenience: A [M,K], B [N,K] (B_NK) or [K,N] (B_KN), same 16-bit dtype on
    one device; C [M,N] allocated by torch when not given.  Returns C."""
    import torch
    if A.dtype not in (torch.float16, torch.bfloat16) or B.dtype != A.dtype:
        raise TypeError("A and B must share dtype float16 or bfloat16")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous (packed row-major)")
    M, K = A.shape
    if b_layout == B_NK:
        N, Kb = B.shape
    else:
        Kb, N = B.shape
    if Kb != K:
        raise ValueError(f"K mismatch: {K} vs {Kb}")
    if C is None:
        C = torch.empty((M, N), dtype=A.dtype, device=A.device)
    elif C.shape != (M, N) or C.dtype != A.dtype or not C.is_contiguous():
        raise ValueError("C must be a contiguous [M,N] tensor of the input dtype")
    dtype = F16 if A.dtype == torch.float16 else BF16
    gemm_ex(dtype, M, N, K, A, B, C, b_layout, config, stream)
    return C
