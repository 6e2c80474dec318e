"""GPU parity at the operand-size limits of the kernels' 32-bit buffer offsets: an
operand of 2^31 bytes (the fast kernels' limit), one just under the masked kernel's
limit (2^31 - 32 bytes) at an odd base address, and one just past it (the generic
kernel).  Inputs are small integers drawn on the device, so every fp32 partial sum is
exact and C must equal the oracle bit for bit; the oracle sees the sampled rows (or
columns) of C that cover the first and last rows and columns of every operand."""
import numpy as np
import pytest

from tests.gpu_util import from_dev, require_gpu, say, torch
from tiled_dense_gemm_major_amd.inputs import BF16, B_KN, B_NK

pytestmark = pytest.mark.gpu

A_MK, A_KM = 0, 1


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _ints(shape, seed, offset=0):
    """A device bf16 tensor of integers in [-2, 2], starting `offset` elements into its
    allocation; returns (allocation, tensor)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    n = int(np.prod(shape))
    flat = torch.empty(n + offset, dtype=torch.bfloat16, device="cuda")
    flat[offset:] = torch.randint(-2, 3, (n,), generator=g, device="cuda",
                                  dtype=torch.int8).to(torch.bfloat16)
    return flat, flat[offset:].view(shape)


def _sample(n, seed):
    rng = np.random.default_rng(seed)
    picks = {0, 1, n // 2, n - 2, n - 1} | set(rng.integers(0, n, 3).tolist())
    return sorted(p for p in picks if 0 <= p < n)


def _configs(b_layout, a_layout, kernel, **match):
    from tiled_dense_gemm_major_amd import tgemm
    out = []
    for c in tgemm.list_configs(BF16, b_layout, a_layout):
        if c.kernel == kernel and all(getattr(c, k) == v for k, v in match.items()):
            out.append(c)
    assert out, (kernel, match)
    return out[:1]


def _run(M, N, K, A, lda, a_layout, B, ldb, b_layout, cfg):
    from tiled_dense_gemm_major_amd import tgemm
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    tgemm.gemm_strided(BF16, M, N, K, A, lda, a_layout, B, ldb, b_layout, C, N, cfg)
    torch.cuda.synchronize()
    return C


def _check_rows(orc, C, A_rows, B_host, b_layout, rows, what):
    want = orc.gemm(BF16, A_rows, B_host, b_layout)
    got = from_dev(C[rows])
    assert np.array_equal(got, want), what


@pytest.mark.parametrize("K,offset,expect", [
    (65536, 0, "fast"),          # A: 2^30 halves = 2^31 bytes, packed, aligned
    (65535, 1, "masked"),        # A: 2^31 - 32768 bytes, odd K, odd base address
])
def test_large_a_mk(dev, orc, K, offset, expect):
    from tiled_dense_gemm_major_amd import tgemm
    M, N = 16384, 256
    _, A = _ints((M, K), 11 + K, offset)
    _, B = _ints((N, K), 12 + K)
    rows = _sample(M, K)
    A_rows = from_dev(A[rows])
    B_host = from_dev(B)
    if expect == "fast":
        cfgs = [None] + _configs(B_NK, A_MK, tgemm.KERNEL_QUAD, block_m=256, mfma=16) \
            + _configs(B_NK, A_MK, tgemm.KERNEL_TILED, block_m=128, block_n=128)
    else:
        cfgs = [None] + _configs(B_NK, A_MK, tgemm.KERNEL_MASKED, block_m=256) \
            + _configs(B_NK, A_MK, tgemm.KERNEL_MASKED, block_m=64)
    for cfg in cfgs:
        say(f"large A [M,K] {M}x{N}x{K} offset {offset} "
            f"{cfg.as_dict() if cfg is not None else 'table choice'}")
        C = _run(M, N, K, A, K, A_MK, B, K, B_NK, cfg)
        _check_rows(orc, C, A_rows, B_host, B_NK, rows, (K, offset, cfg))
    if expect == "masked":
        assert tgemm.query_config(BF16, M, N, K, B_NK, False).kernel == tgemm.KERNEL_MASKED


def test_large_a_past_masked_limit(dev, orc):
    """A of 2^31 + 98 302 bytes (odd K): past both buffer limits, the generic kernel."""
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 16385, 256, 65535
    _, A = _ints((M, K), 21)
    _, B = _ints((N, K), 22)
    rows = _sample(M, 23)
    say(f"large A past the masked limit {M}x{N}x{K}: table choice")
    C = _run(M, N, K, A, K, A_MK, B, K, B_NK, None)
    _check_rows(orc, C, from_dev(A[rows]), from_dev(B), B_NK, rows, "generic")
    # an explicit masked configuration is refused for it
    cfg = _configs(B_NK, A_MK, tgemm.KERNEL_MASKED, block_m=128, block_n=128)[0]
    with pytest.raises(tgemm.TGemmError):
        _run(M, N, K, A, K, A_MK, B, K, B_NK, cfg)


@pytest.mark.parametrize("N,expect", [
    (16384, "fast"),             # B [K,N]: 2^30 halves = 2^31 bytes
    (16383, "masked"),           # B [K,N]: 2^31 - 131 072 bytes, odd N
])
def test_large_b_kn(dev, orc, N, expect):
    from tiled_dense_gemm_major_amd import tgemm
    M, K = 256, 65536
    _, A = _ints((M, K), 31 + N)
    _, B = _ints((K, N), 32 + N)
    cols = _sample(N, N)
    A_host = from_dev(A)
    B_cols = from_dev(B[:, cols])                      # [K, len(cols)]
    if expect == "fast":
        cfgs = [None] + _configs(B_KN, A_MK, tgemm.KERNEL_QUAD)
    else:
        cfgs = [None] + _configs(B_KN, A_MK, tgemm.KERNEL_MASKED, block_m=64)
    want = orc.gemm(BF16, A_host, B_cols, B_KN)
    for cfg in cfgs:
        say(f"large B [K,N] {M}x{N}x{K} {cfg.as_dict() if cfg is not None else 'table choice'}")
        C = _run(M, N, K, A, K, A_MK, B, N, B_KN, cfg)
        assert np.array_equal(from_dev(C[:, cols]), want), (N, cfg)


def test_large_a_km(dev, orc):
    """A stored [K,M] at 2^31 bytes (the quad kernel's transposing A reads)."""
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 16384, 256, 65536
    _, A = _ints((K, M), 41)                            # storage [K,M], lda = M
    _, B = _ints((N, K), 42)
    rows = _sample(M, 43)
    A_rows = np.ascontiguousarray(from_dev(A[:, rows]).T)   # logical rows [R, K]
    B_host = from_dev(B)
    for cfg in [None] + _configs(B_NK, A_KM, tgemm.KERNEL_QUAD):
        say(f"large A [K,M] {M}x{N}x{K} {cfg.as_dict() if cfg is not None else 'table choice'}")
        C = _run(M, N, K, A, M, A_KM, B, K, B_NK, cfg)
        _check_rows(orc, C, A_rows, B_host, B_NK, rows, cfg)
