"""Seeded synthetic inputs for the GEMM: the one module both the GPU path and the CPU oracle
are fed from.  It holds no part of the product's arithmetic -- only random draws and the
rounding of each draw to a 16-bit input format.

Recipe (the same for every caller, so a workload is fixed by its name and seed):

* Random stream: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014; the generator ``splitmix64`` of S. Vigna).  Draw ``i``
  (0-based) of seed ``s`` is ``mix(s + (i+1) * 0x9E3779B97F4A7C15)`` with the published
  mixing constants, so any range of draws can be produced independently of the rest.
* U[0,1): the top 53 bits of a draw times 2^-53.
* uniform[-1,1): 2*U - 1 (exact in fp64).
* normal(0, sigma): Box-Muller (Box & Muller, 1958) on a pair of draws (u1 = 1 - U in
  (0,1], u2 = U): r = sqrt(-2 ln u1), values r*cos(2 pi u2) and r*sin(2 pi u2), both kept,
  in that order, each times sigma (sigma is the standard deviation).
* Rounding to the input format: round-to-nearest-even from the fp64 draw -- numpy's
  float64 -> float16 conversion for fp16; for bf16 an integer rounding of the fp64 bit
  pattern to 7 fraction bits (valid for the normal bf16 range, which every draw here is in).
* A workload fills A in its storage order first, then B in its storage order, from one
  stream.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F16, BF16 = 0, 1
B_NK, B_KN = 0, 1
DTYPE_NAMES = {F16: "f16", BF16: "bf16"}

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 23


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Draws [start, start+count) of the SplitMix64 stream of ``seed`` (uint64)."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _unit(draws: np.ndarray) -> np.ndarray:
    return (draws >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def round_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16, nearest-even, for values that are zero or in the normal bf16 range."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    if np.any((mag != 0) & ((mag < 2.0 ** -126) | (mag >= 2.0 ** 127))):
        raise ValueError("draw outside the normal bf16 range")
    u = x.view(np.uint64)
    drop = np.uint64(52 - 7)                       # fp64 fraction bits below bf16's seven
    lsb = (u >> drop) & np.uint64(1)
    r = (u + (np.uint64(1) << (drop - np.uint64(1))) - np.uint64(1) + lsb)
    r &= ~((np.uint64(1) << drop) - np.uint64(1))  # now exactly a bf16 value, held in fp64
    f32 = r.view(np.float64).astype(np.float32)    # exact: 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


class Stream:
    """Sequential consumer of one seed's draws."""

    def __init__(self, seed: int):
        self.seed = seed
        self.pos = 0

    def _take(self, count: int) -> np.ndarray:
        out = splitmix64(self.seed, self.pos, count)
        self.pos += count
        return out

    def unit(self, count: int) -> np.ndarray:
        """U[0,1) doubles (53 random bits each)."""
        return _unit(self._take(count))

    def uniform_pm1(self, count: int) -> np.ndarray:
        return 2.0 * _unit(self._take(count)) - 1.0

    def normal(self, count: int, sigma: float) -> np.ndarray:
        pairs = (count + 1) // 2
        d = self._take(2 * pairs)
        u1 = 1.0 - _unit(d[0::2])
        u2 = _unit(d[1::2])
        r = np.sqrt(-2.0 * np.log(u1))
        z = np.empty(2 * pairs, dtype=np.float64)
        z[0::2] = r * np.cos(2.0 * np.pi * u2)
        z[1::2] = r * np.sin(2.0 * np.pi * u2)
        return sigma * z[:count]

    def matrix(self, shape, dtype: int, dist: str, sigma: float = 0.5) -> np.ndarray:
        """A matrix of 16-bit patterns filled in storage (row-major) order."""
        count = int(np.prod(shape))
        out = np.empty(count, dtype=np.uint16)
        rnd = round_to_f16_bits if dtype == F16 else round_to_bf16_bits
        done = 0
        while done < count:
            c = min(_CHUNK, count - done)
            if dist == "uniform":
                x = self.uniform_pm1(c)
            elif dist == "normal":
                if c % 2 and done + c < count:
                    raise AssertionError("normal chunks must be even")
                x = self.normal(c, sigma)
            else:
                raise ValueError(f"unknown distribution {dist!r}")
            out[done:done + c] = rnd(x)
            done += c
        return out.reshape(shape)


@dataclass(frozen=True)
class Workload:
    """One GEMM workload: C[M,N] = sum_k A[M,K] * B(N,K)."""
    name: str
    dtype: int
    M: int
    N: int
    K: int
    b_layout: int
    dist: str
    seed: int
    sigma: float = 0.5

    @property
    def a_shape(self):
        return (self.M, self.K)

    @property
    def b_shape(self):
        return (self.N, self.K) if self.b_layout == B_NK else (self.K, self.N)

    def generate(self):
        """(A bits [M,K], B bits in its storage shape), both uint16."""
        s = Stream(self.seed)
        A = s.matrix(self.a_shape, self.dtype, self.dist, self.sigma)
        B = s.matrix(self.b_shape, self.dtype, self.dist, self.sigma)
        return A, B

    def describe(self) -> str:
        lay = "B[N,K]" if self.b_layout == B_NK else "B[K,N]"
        d = "U[-1,1]" if self.dist == "uniform" else f"N(0,{self.sigma})"
        return (f"{DTYPE_NAMES[self.dtype]} {self.M}x{self.N}x{self.K} {lay} {d} "
                f"seed {self.seed}")


# The five workloads: shapes, layouts and value distributions of the pages' problem
# (the K-major C = A x B^T at 512^3, 4096^3 and 8192^3, a ragged N-major-B case and a
# skinny decode-like case).
WORKLOADS = {
    "f16_512": Workload("f16_512", F16, 512, 512, 512, B_NK, "uniform", 1),
    "bf16_4096": Workload("bf16_4096", BF16, 4096, 4096, 4096, B_NK, "uniform", 2),
    "bf16_8192": Workload("bf16_8192", BF16, 8192, 8192, 8192, B_NK, "uniform", 3),
    "f16_4000x3000x1000_kn": Workload("f16_4000x3000x1000_kn", F16, 4000, 3000, 1000, B_KN,
                                      "normal", 4, 0.5),
    "bf16_skinny_64x8192x8192": Workload("bf16_skinny_64x8192x8192", BF16, 64, 8192, 8192,
                                         B_NK, "uniform", 5),
}


@dataclass(frozen=True)
class AttnWorkload:
    """One attention-forward workload: Q, K, V, O of shape [batch, seq, heads, dim], fp16
    ("TileLang: a tile language one level below Triton", section "FlashAttention: online
    softmax as tile code": (batch, seq, heads, dim) tensors in float16, causal mask)."""
    name: str
    batch: int
    seq: int
    heads: int
    dim: int
    causal: bool
    seed: int
    dist: str = "normal"
    sigma: float = 1.0

    @property
    def shape(self):
        return (self.batch, self.seq, self.heads, self.dim)

    def describe(self) -> str:
        return (f"fp16 attention B={self.batch} S={self.seq} H={self.heads} D={self.dim} "
                f"{'causal' if self.causal else 'full'} N(0,{self.sigma:g}) seed {self.seed}")

    def generate(self):
        """(Q, K, V) bits, uint16 [B, S, H, D], filled in that order."""
        s = Stream(self.seed)
        return tuple(s.matrix(self.shape, F16, self.dist, self.sigma) for _ in range(3))


ATTN_WORKLOADS = {
    # the page's configuration: flash_attn(1, 8, 1024, 64), causal
    "attn_f16_b1_s1024_h8_d64_causal": AttnWorkload("attn_f16_b1_s1024_h8_d64_causal",
                                                    1, 1024, 8, 64, True, 6),
    # a larger one of the same kind, for throughput
    "attn_f16_b4_s4096_h16_d64_causal": AttnWorkload("attn_f16_b4_s4096_h16_d64_causal",
                                                     4, 4096, 16, 64, True, 7),
}

