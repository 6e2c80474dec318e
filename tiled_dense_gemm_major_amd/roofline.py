"""Work and traffic model of the tiled GEMM, and the MI355X ceilings it is measured against.

The counting follows "Tiling a matmul" (H. Sonawane), section "Counting traffic": a
product of N x N matrices does 2N^3 floating-point operations; with T x T output tiles
every tile reads a T-row strip of A and a T-column strip of B, so the inputs are read
N/T times each (2N^3/T elements) and the output is written once (N^2 elements); in a
16-bit format the intensity is about T/2 FLOP per byte.  The rectangular form (the
exercise in section "Try it") reads M*N*K*(1/BN + 1/BM) input elements.  The compulsory
traffic -- every input read once, the output written once -- is the floor a good launch
order approaches through cache reuse (section "The levels of tiling").

The shared-memory arithmetic follows the same page (section "Shared memory sets the
ceiling") and the exercises of "TileLang: a tile language one level below Triton": one
pipeline stage holds an A tile and a B tile; the stages multiply it.
"""
from __future__ import annotations

# MI355X published peaks (dense, no sparsity).
PEAK_FLOPS = {"f16": 2.5e15, "bf16": 2.5e15}
HBM_BYTES_PER_S = 8.0e12
LDS_BYTES_PER_CU = 160 * 1024
NUM_CUS = 256


def gemm_flops(M: int, N: int, K: int) -> int:
    """2*M*N*K: one multiply and one add per (m, n, k)."""
    return 2 * M * N * K


def compulsory_bytes(M: int, N: int, K: int, elem: int = 2) -> int:
    """A and B read once, C written once."""
    return elem * (M * K + N * K + M * N)


def square_tile_traffic_bytes(n: int, t: int, elem: int = 2) -> int:
    """No-cache traffic of an n x n product with t x t tiles, in bytes: elem * (2 n^3 / t
    + n^2) -- the n^2 / t^2 tiles each stream a t-row strip of A and a t-column strip of
    B (2 t n elements), and C is written once."""
    return elem * (2 * n ** 3 // t + n * n)


def tile_traffic_bytes(M: int, N: int, K: int, bm: int, bn: int, elem: int = 2) -> int:
    """No-cache traffic with bm x bn output tiles (ragged edges counted as whole tiles)."""
    tm = -(-M // bm)
    tn = -(-N // bn)
    reads = tm * tn * (bm + bn) * K
    return (reads + M * N) * elem


def stage_bytes(bm: int, bn: int, bk: int, elem: int = 2) -> int:
    """One pipeline stage: an A tile [bm, bk] and a B tile [bn, bk]."""
    return (bm + bn) * bk * elem


def pipeline_bytes(bm: int, bn: int, bk: int, stages: int, elem: int = 2) -> int:
    return stages * stage_bytes(bm, bn, bk, elem)


def blocks_per_unit(smem_per_block: int, smem_per_unit: int) -> int:
    """How many blocks of this footprint one unit of that capacity holds."""
    return smem_per_unit // smem_per_block


def roofline_time_s(M: int, N: int, K: int, dtype: str = "bf16") -> float:
    return max(gemm_flops(M, N, K) / PEAK_FLOPS[dtype],
               compulsory_bytes(M, N, K) / HBM_BYTES_PER_S)


def bound(M: int, N: int, K: int, dtype: str = "bf16") -> str:
    """'mfma' when the compulsory intensity is above the ridge, else 'hbm'."""
    ai = gemm_flops(M, N, K) / compulsory_bytes(M, N, K)
    return "mfma" if ai >= PEAK_FLOPS[dtype] / HBM_BYTES_PER_S else "hbm"


def attention_flops(batch: int, seq: int, heads: int, dim: int, causal: bool) -> int:
    """Attention forward: the multiply-adds of Q K^T and of P V (two flops each) over the
    (query, key) pairs the mask keeps -- seq*(seq+1)/2 per (batch, head) when causal
    ("TileLang: a tile language one level below Triton", exercise 3: causal attention
    does about half the work of full attention), seq*seq otherwise."""
    pairs = seq * (seq + 1) // 2 if causal else seq * seq
    return 4 * batch * heads * pairs * dim


def attention_bytes(batch: int, seq: int, heads: int, dim: int, elem: int = 2) -> int:
    """Compulsory traffic: Q, K, V read once, O written once."""
    return 4 * batch * seq * heads * dim * elem

