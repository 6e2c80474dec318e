"""CPU oracle for the block-tiled dense GEMM -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of ``bench.py`` may import
this package.  It shares no code with the GPU library: ``oracle.c`` is built here with gcc
and loaded with ctypes.

What the oracle computes is stated in ``oracle.c``: the plain sum over k of the exact
fp16/bf16 input products, accumulated in fp64 in increasing k and rounded once, to
nearest-even, to the 16-bit output format.  Sources: "0. A Minimal Hopper Matmul" (Tilus
tutorial), section "Block Tiling" (C = A x B^T, A (M,K), B (N,K)); "Tiling a matmul",
section "Code" (the naive sum with B indexed [k][j]); "TileLang: a tile language one level
below Triton", section "The first kernel: GEMM" (B as a (K,N) tensor).

The acceptance test that the GPU results are held to (``tolerance`` below) allows, per
element, 1e-3 * sqrt(K) plus one step ("ulp") of the output format at the oracle's value.

``attention`` is the plain definition of the attention forward pass of "TileLang: a tile
language one level below Triton", section "FlashAttention: online softmax as tile code"
(softmax over the keys of Q K^T / sqrt(dim), causal or not, times V; fp64, one rounding to
fp16); ``attention_tolerance`` states the bound its GPU results are held to.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F16, BF16 = 0, 1
B_NK, B_KN = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra"]


def build() -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_max_threads.restype = i32
    lib.oracle_decode.argtypes = [i32, vp, vp, i64]
    lib.oracle_encode.argtypes = [i32, vp, vp, i64]
    lib.oracle_gemm.argtypes = [i32, i64, i64, i64, vp, vp, i32, vp, vp, i32]
    lib.oracle_gemm_rows.argtypes = [i32, i64, i64, i64, vp, vp, i32, i64, i64, vp, vp, i32]
    lib.oracle_gemm_entries.argtypes = [i32, i64, i64, i64, vp, vp, i32, i64, vp, vp, vp, vp,
                                        i32]
    lib.oracle_gemm_f64.argtypes = [i64, i64, i64, vp, vp, i32, vp, i32]
    lib.oracle_tiled_f64.argtypes = [i64, i64, vp, vp, vp, vp]
    lib.oracle_attention.argtypes = [i64, i64, i64, i64, vp, vp, vp, i32, vp, vp, i32]
    for name in ("oracle_decode", "oracle_encode", "oracle_gemm", "oracle_gemm_rows",
                 "oracle_gemm_entries", "oracle_gemm_f64", "oracle_tiled_f64",
                 "oracle_attention"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {a.dtype}")
    return a


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def decode(dtype: int, bits) -> np.ndarray:
    """16-bit patterns -> exact fp64 values."""
    bits = _u16(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    _check(_load().oracle_decode(dtype, _ptr(bits), _ptr(out), bits.size), "decode")
    return out


def encode(dtype: int, values) -> np.ndarray:
    """fp64 values -> 16-bit patterns, round to nearest even (one rounding)."""
    values = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(values.shape, dtype=np.uint16)
    _check(_load().oracle_encode(dtype, _ptr(values), _ptr(out), values.size), "encode")
    return out


def _dims(A, B, b_layout):
    M, K = A.shape
    if b_layout == B_NK:
        N, Kb = B.shape
    elif b_layout == B_KN:
        Kb, N = B.shape
    else:
        raise ValueError(f"bad b_layout {b_layout}")
    if Kb != K:
        raise ValueError(f"K mismatch: A has {K}, B has {Kb}")
    return M, N, K


def gemm(dtype: int, A, B, b_layout: int = B_NK, nthreads: int = 0, want_sums=False):
    """The whole product.  A: uint16 [M,K]; B: uint16 [N,K] (NK) or [K,N] (KN).
    Returns the rounded C bits [M,N] (and the fp64 sums if ``want_sums``)."""
    A, B = _u16(A), _u16(B)
    M, N, K = _dims(A, B, b_layout)
    C = np.empty((M, N), dtype=np.uint16)
    S = np.empty((M, N), dtype=np.float64) if want_sums else None
    _check(_load().oracle_gemm(dtype, M, N, K, _ptr(A), _ptr(B), b_layout, _ptr(C), _ptr(S),
                               nthreads), "gemm")
    return (C, S) if want_sums else C


def gemm_rows(dtype: int, A, B, b_layout: int, m_lo: int, m_hi: int, nthreads: int = 0):
    """Rows [m_lo, m_hi) of C (rounded bits)."""
    A, B = _u16(A), _u16(B)
    M, N, K = _dims(A, B, b_layout)
    C = np.empty((m_hi - m_lo, N), dtype=np.uint16)
    _check(_load().oracle_gemm_rows(dtype, M, N, K, _ptr(A), _ptr(B), b_layout, m_lo, m_hi,
                                    _ptr(C), None, nthreads), "gemm_rows")
    return C


def gemm_entries(dtype: int, A, B, b_layout: int, rows, cols, nthreads: int = 0):
    """C at the positions (rows[i], cols[i]), each summed on its own.
    Returns (rounded bits, fp64 sums)."""
    A, B = _u16(A), _u16(B)
    M, N, K = _dims(A, B, b_layout)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in shape")
    C = np.empty(rows.shape, dtype=np.uint16)
    S = np.empty(rows.shape, dtype=np.float64)
    _check(_load().oracle_gemm_entries(dtype, M, N, K, _ptr(A), _ptr(B), b_layout, rows.size,
                                       _ptr(rows), _ptr(cols), _ptr(C), _ptr(S), nthreads),
           "gemm_entries")
    return C, S


def gemm_f64(A, B, b_layout: int = B_NK, nthreads: int = 0) -> np.ndarray:
    """The fp64 sums of fp64 operands (no 16-bit rounding anywhere)."""
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    M, K = A.shape
    N = B.shape[0] if b_layout == B_NK else B.shape[1]
    S = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_gemm_f64(M, N, K, _ptr(A), _ptr(B), b_layout, _ptr(S), nthreads),
           "gemm_f64")
    return S


def tiled_f64(A, B, t: int):
    """The square tiled loop of "Tiling a matmul" (B stored [K,N]).  Returns (C, loads)."""
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    n = A.shape[0]
    C = np.empty((n, n), dtype=np.float64)
    loads = ctypes.c_int64(0)
    _check(_load().oracle_tiled_f64(n, t, _ptr(A), _ptr(B), _ptr(C), ctypes.byref(loads)),
           "tiled_f64")
    return C, int(loads.value)


def attention(Q, K, V, causal: bool, nthreads: int = 0, want_f64: bool = False):
    """Attention forward on fp16 bit patterns [B, S, H, D] (the definition in oracle.c:
    softmax over the keys of Q K^T / sqrt(D), causal or not, times V; one rounding).
    Returns O's bits (and the unrounded fp64 values if ``want_f64``)."""
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    if Q.ndim != 4 or Q.shape != K.shape or Q.shape != V.shape:
        raise ValueError("Q, K, V must share one [B, S, H, D] shape")
    Bn, S, H, D = Q.shape
    O = np.empty(Q.shape, dtype=np.uint16)
    O64 = np.empty(Q.shape, dtype=np.float64) if want_f64 else None
    _check(_load().oracle_attention(Bn, S, H, D, _ptr(Q), _ptr(K), _ptr(V), int(bool(causal)),
                                    _ptr(O), _ptr(O64), nthreads), "attention")
    return (O, O64) if want_f64 else O


def attention_tolerance(V, causal: bool, orc_values) -> np.ndarray:
    """Per-element bound for a kernel that rounds the softmax weights to fp16 before the
    product with V (as the page's kernel does) and sums those rounded weights for the
    normalizer: each weight is off by at most 2^-11 relative, so the normalized average
    moves by at most 2 * 2^-11 * max_j |v(j,d)| over the keys it averages; doubled for
    the fp32 score, exponential and sum errors, plus one fp16 ulp of |oracle| for the two
    final roundings.  max_j |v(j,d)| is taken over all keys of the (batch, head) (a
    superset of the keys a causal row sees)."""
    v = np.abs(decode(F16, V))                              # [B, S, H, D]
    vmax = v.max(axis=1, keepdims=True)                     # [B, 1, H, D]
    return 4.0 * 2.0 ** -11 * np.broadcast_to(vmax, v.shape) + ulp_out(F16, orc_values)


def compare_attention(V, causal: bool, got_bits, want_bits) -> dict:
    got = decode(F16, got_bits)
    want = decode(F16, want_bits)
    tol = attention_tolerance(V, causal, want)
    err = np.abs(got - want)
    bad = ~np.isfinite(got) | ~(err <= tol)
    idx = np.flatnonzero(bad.ravel())
    return {
        "n": int(got.size),
        "n_fail": int(idx.size),
        "first_fail": int(idx[0]) if idx.size else -1,
        "max_err": float(np.max(err)) if err.size else 0.0,
        "max_err_over_tol": float(np.max(err / tol)) if err.size else 0.0,
    }


# ---------------------------------------------------------------------------------------
# The acceptance rule for GPU results.
# ---------------------------------------------------------------------------------------
_PRECISION = {F16: 11, BF16: 8}            # significand bits including the hidden one
_MIN_NORMAL_EXP = {F16: -14, BF16: -126}


def ulp_out(dtype: int, x) -> np.ndarray:
    """Spacing of the output format at |x|: 2^(floor(log2|x|) - p + 1) in the normal range,
    the subnormal spacing 2^(emin - p + 1) below it and at zero (2^-24 for fp16, 2^-133
    for bf16).  A non-finite x has no spacing: NaN, so no comparison against it passes."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    p = _PRECISION[dtype]
    emin = _MIN_NORMAL_EXP[dtype]
    _, e = np.frexp(x)                      # x = f * 2^e, f in [0.5, 1); frexp(0) gives e = 0
    floor_log2 = np.where(x == 0.0, emin, e.astype(np.int64) - 1)
    expo = np.maximum(floor_log2, emin) - (p - 1)
    return np.where(np.isfinite(x), np.ldexp(1.0, expo), np.nan)


def tolerance(dtype: int, K: int, orc_values) -> np.ndarray:
    """Per-element bound: 1e-3 * sqrt(K) + one output-format ulp of |oracle|."""
    return 1e-3 * np.sqrt(float(K)) + ulp_out(dtype, orc_values)


def compare(dtype: int, K: int, got_bits, want_bits) -> dict:
    """Element-wise check of 16-bit results against the oracle's 16-bit results."""
    got = decode(dtype, got_bits).ravel()
    want = decode(dtype, want_bits).ravel()
    tol = tolerance(dtype, K, want)
    with np.errstate(invalid="ignore"):        # inf - inf is NaN: a failure below
        err = np.abs(got - want)
    bad = ~np.isfinite(got) | ~(err <= tol)
    idx = np.flatnonzero(bad)
    ratio = np.where(np.isfinite(err), err / tol, np.inf)
    return {
        "n": int(got.size),
        "n_fail": int(idx.size),
        "first_fail": int(idx[0]) if idx.size else -1,
        "max_err": float(np.max(err)) if err.size else 0.0,
        "max_err_over_tol": float(np.max(ratio)) if ratio.size else 0.0,
    }
