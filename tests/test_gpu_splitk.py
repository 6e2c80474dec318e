"""GPU parity of split-K over workgroups (gemm_ex_ws with a lent workspace): the K range
of each C tile summed by several workgroups into fp32 partial tiles, then added in split
order and cast once.  Held to the oracle's rule element by element; bit for bit where
every partial sum is exact; the same bits on every launch (fixed order, no atomics)."""
import numpy as np
import pytest

from tests.gpu_util import (assert_parity, from_dev, require_gpu, say,
                            tdtype, to_dev, torch)
from tiled_dense_gemm_major_amd.inputs import BF16, B_KN, B_NK, F16, WORKLOADS, Stream

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _splitk(splits, block_n=256):
    from tiled_dense_gemm_major_amd import tgemm
    return tgemm.Config(kernel=tgemm.KERNEL_SPLITK, block_m=64, block_n=block_n, block_k=32,
                        waves_m=1, waves_n=4, stages=5, group_m=1, split_k=splits, mfma=32)


def _run_ws(dtype, A, B, cfg, ws_fill=-1, guard=1024):
    """C from gemm_ex_ws; the workspace (pre-filled with ws_fill) has a guard band after
    the bytes the configuration needs, which must stay untouched."""
    from tiled_dense_gemm_major_amd import tgemm
    M, K = A.shape
    N = B.shape[0]
    need = tgemm.workspace_size(M, N, cfg) if cfg is not None else \
        tgemm.query_config_ws(dtype, M, N, K)[1]
    ws = torch.full(((need + guard) // 4,), ws_fill, dtype=torch.int32, device="cuda")
    C = torch.full((M, N), 0x7E00, dtype=torch.int16, device="cuda").view(tdtype(dtype))
    tgemm.gemm_ex_ws(dtype, M, N, K, to_dev(A, dtype), to_dev(B, dtype), C, ws, need, B_NK,
                     cfg)
    torch.cuda.synchronize()
    host = ws.cpu().numpy()
    assert np.all(host[need // 4:] == ws_fill), "workspace written past its size"
    return from_dev(C)


def _inputs(dtype, M, N, K, seed):
    s = Stream(seed)
    return s.matrix((M, K), dtype, "uniform"), s.matrix((N, K), dtype, "uniform")


def _int_bits(dtype, vals):
    from tiled_dense_gemm_major_amd.inputs import round_to_bf16_bits, round_to_f16_bits
    f = round_to_f16_bits if dtype == F16 else round_to_bf16_bits
    return f(np.asarray(vals, dtype=np.float64))


_WANT = {}


def _case(orc, dtype, M, N, K):
    """Seeded inputs and the oracle's product for one (dtype, shape), computed once."""
    key = (dtype, M, N, K)
    if key not in _WANT:
        A, B = _inputs(dtype, M, N, K, 11 + M + N + K)
        _WANT[key] = (A, B, orc.gemm(dtype, A, B, B_NK))
    return _WANT[key]


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("shape", [(64, 1024, 2048), (50, 1000, 3000), (1, 264, 1032),
                                   (128, 520, 4104), (200, 536, 328)])
@pytest.mark.parametrize("splits", [2, 3, 8, 13, 64])
@pytest.mark.parametrize("block_n", [256, 128])
def test_splitk_ragged(dev, orc, dtype, shape, splits, block_n):
    M, N, K = shape
    A, B, want = _case(orc, dtype, M, N, K)
    say(f"split-K {dtype} {shape} splits {splits} block_n {block_n}")
    got = _run_ws(dtype, A, B, _splitk(splits, block_n))
    assert_parity(orc, dtype, K, got, want, f"split-K {shape} x{splits}")


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("K", [0, 8, 72, 200, 1000, 2056])
def test_splitk_exact_small_integers(dev, orc, dtype, K):
    """Small-integer inputs make every partial sum exact: any split must give the oracle's
    bits, including splits with nothing to sum (K shorter than the splits)."""
    rng = np.random.default_rng(K + 5)
    M, N = 72, 520
    A = _int_bits(dtype, rng.integers(-2, 3, (M, K)))
    B = _int_bits(dtype, rng.integers(-2, 3, (N, K)))
    want = orc.gemm(dtype, A, B, B_NK)
    if K == 0:
        # packed operands with K = 0 have lda = 1, which no fast configuration takes: the
        # table's choice (the generic kernel) writes the empty sums, with a workspace lent
        say(f"split-K entry point K=0 {dtype}")
        assert np.array_equal(_run_ws(dtype, A, B, None), want)
        return
    for splits in (2, 5, 8, 32):
        say(f"split-K exact {dtype} K={K} splits {splits}")
        assert np.array_equal(_run_ws(dtype, A, B, _splitk(splits)), want), (K, splits)


def test_splitk_table_choice_skinny_workload(dev, orc):
    """The skinny workload at full size through the table's choice with a workspace
    (the split-K kernel), every element against the oracle."""
    from tiled_dense_gemm_major_amd import tgemm
    w = WORKLOADS["bf16_skinny_64x8192x8192"]
    cfg, need = tgemm.query_config_ws(w.dtype, w.M, w.N, w.K)
    assert cfg.kernel == tgemm.KERNEL_SPLITK and need > 0
    A, B = w.generate()
    say(f"split-K table choice {w.describe()} splits {cfg.split_k}")
    got = _run_ws(w.dtype, A, B, None)
    assert not np.any(got == 0x7E00)
    assert_parity(orc, w.dtype, w.K, got, orc.gemm(w.dtype, A, B, w.b_layout),
                  "skinny split-K")


def test_splitk_table_choice_wide_skinny(dev, orc):
    """A skinny product with more than 128 tiles of 64x128 (ragged N) on the split-K
    kernel's 64x256 tiles, 2 splits, every element against the oracle; with a workspace
    the table itself keeps the skinny kernel's plain 64-column form here."""
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 48, 28680, 2056
    table, need = tgemm.query_config_ws(BF16, M, N, K)
    assert (table.kernel, table.block_n, need) == (tgemm.KERNEL_SKINNY, 64, 0)
    cfg = tgemm.Config(kernel=tgemm.KERNEL_SPLITK, block_m=64, block_n=256, block_k=64,
                       waves_m=1, waves_n=4, stages=4, group_m=1, split_k=2, mfma=32)
    assert tgemm.workspace_size(M, N, cfg) == 2 * M * N * 4
    A, B, want = _case(orc, BF16, M, N, K)
    say(f"split-K bf16 {M}x{N}x{K}: 64x256 tiles, 2 splits")
    got = _run_ws(BF16, A, B, cfg)
    assert not np.any(got == 0x7E00)
    assert_parity(orc, BF16, K, got, want, "wide skinny split-K")


def test_splitk_repeat_launches_bitwise_identical(dev, orc):
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 96, 4096, 8192
    A, B = _inputs(BF16, M, N, K, 23)
    Ad, Bd = to_dev(A, BF16), to_dev(B, BF16)
    cfg = _splitk(16)
    need = tgemm.workspace_size(M, N, cfg)
    ws = torch.empty((need // 4,), dtype=torch.int32, device="cuda")
    C0 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    tgemm.gemm_ex_ws(BF16, M, N, K, Ad, Bd, C0, ws, need, B_NK, cfg)
    torch.cuda.synchronize()
    ref = from_dev(C0)
    assert_parity(orc, BF16, K, ref, orc.gemm(BF16, A, B, B_NK), "split-K")
    say("split-K repeat launches")
    C = torch.empty_like(C0)
    for _ in range(20):
        tgemm.gemm_ex_ws(BF16, M, N, K, Ad, Bd, C, ws, need, B_NK, cfg)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(C), ref)


def test_splitk_does_not_write_outside_c(dev, orc):
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 70, 264, 1032
    A, B = _inputs(F16, M, N, K, 4)
    guard = 4096
    buf = torch.full((guard + M * N + guard,), 0x1234, dtype=torch.int16, device="cuda")
    C = buf[guard:guard + M * N].view(torch.float16).view(M, N)
    cfg = _splitk(8)
    need = tgemm.workspace_size(M, N, cfg)
    ws = torch.empty((need // 4,), dtype=torch.int32, device="cuda")
    say("split-K guard bands")
    tgemm.gemm_ex_ws(F16, M, N, K, to_dev(A, F16), to_dev(B, F16), C, ws, need, B_NK, cfg)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:guard] == 0x1234) and np.all(host[guard + M * N:] == 0x1234)
    assert_parity(orc, F16, K, host[guard:guard + M * N].view(np.uint16).reshape(M, N),
                  orc.gemm(F16, A, B, B_NK), "split-K guard")


def test_splitk_one_workspace_many_shapes(dev, orc):
    """One workspace through a sequence of different shapes and split counts: what a call
    leaves behind must not leak into the next."""
    from tiled_dense_gemm_major_amd import tgemm
    shapes = [(64, 1024, 2048, 8), (128, 2048, 1032, 4), (8, 264, 4104, 16), (64, 1024, 2048, 3),
              (200, 536, 328, 64)]
    need = max(tgemm.workspace_size(M, N, _splitk(sk)) for M, N, K, sk in shapes)
    ws = torch.empty((need // 4,), dtype=torch.int32, device="cuda")
    for rep in range(2):
        for M, N, K, sk in shapes:
            A, B, want = _case(orc, BF16, M, N, K)
            C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            say(f"one workspace {M}x{N}x{K} splits {sk} pass {rep}")
            tgemm.gemm_ex_ws(BF16, M, N, K, to_dev(A, BF16), to_dev(B, BF16), C, ws, need,
                             B_NK, _splitk(sk))
            torch.cuda.synchronize()
            assert_parity(orc, BF16, K, from_dev(C), want, f"{M}x{N}x{K} x{sk}")


# ---------------------------------------------------------------------------------------
# The quad kernel in split-K mode (TGEMM_KERNEL_QUAD_SPLITK): 256x256 tiles, each K range
# of kc (a multiple of 64) walked by the unchanged quad K walk on shifted operands, fp32
# partial tiles, the same fixed-order reduction.
# ---------------------------------------------------------------------------------------
def _quad_split(layout, splits):
    from tiled_dense_gemm_major_amd import tgemm
    return tgemm.Config(kernel=tgemm.KERNEL_QUAD_SPLITK, block_m=256, block_n=256, block_k=64,
                        waves_m=2, waves_n=2, stages=5, group_m=4, split_k=splits,
                        mfma=16 if layout == B_NK else 32)


def _run_quad_split(dtype, A, B, layout, splits, guard=1024):
    """C from gemm_ex_ws with the quad split-K kernel; the workspace is pre-filled with a
    NaN pattern and has a guard band after the bytes the configuration needs."""
    from tiled_dense_gemm_major_amd import tgemm
    M, K = A.shape
    N = B.shape[0] if layout == B_NK else B.shape[1]
    cfg = _quad_split(layout, splits)
    need = tgemm.workspace_size(M, N, cfg)
    assert need == splits * M * N * 4
    ws = torch.full(((need + guard) // 4,), -1, dtype=torch.int32, device="cuda")
    C = torch.full((M, N), 0x7E00, dtype=torch.int16, device="cuda").view(tdtype(dtype))
    tgemm.gemm_ex_ws(dtype, M, N, K, to_dev(A, dtype), to_dev(B, dtype), C, ws, need, layout,
                     cfg)
    torch.cuda.synchronize()
    assert np.all(ws.cpu().numpy()[need // 4:] == -1), "workspace written past its size"
    return from_dev(C)


def _layout_inputs(dtype, M, N, K, layout, seed, ints=False):
    if ints:
        rng = np.random.default_rng(seed)
        A = _int_bits(dtype, rng.integers(-2, 3, (M, K)))
        B = _int_bits(dtype, rng.integers(-2, 3, (N, K) if layout == B_NK else (K, N)))
        return A, B
    s = Stream(seed)
    return (s.matrix((M, K), dtype, "uniform"),
            s.matrix((N, K) if layout == B_NK else (K, N), dtype, "uniform"))


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("layout", [B_NK, B_KN])
@pytest.mark.parametrize("shape", [(600, 536, 1000), (300, 520, 4104), (257, 264, 328),
                                   (64, 1024, 2048)])
def test_quad_split_ragged(dev, orc, dtype, layout, shape):
    """Ragged tiles, a K tail in the last range, and split counts that leave the last
    range short or (for the short K) several ranges empty."""
    M, N, K = shape
    A, B = _layout_inputs(dtype, M, N, K, layout, 500 + M + N + K + layout)
    want = orc.gemm(dtype, A, B, layout)
    for splits in (2, 3, 5, 16):
        say(f"quad split-K {dtype} layout {layout} {shape} splits {splits}")
        got = _run_quad_split(dtype, A, B, layout, splits)
        assert_parity(orc, dtype, K, got, want, f"quad split-K {shape} x{splits}")


@pytest.mark.parametrize("layout", [B_NK, B_KN])
@pytest.mark.parametrize("K", [8, 64, 200, 1000, 1032, 4104])
def test_quad_split_exact_ints(dev, orc, layout, K):
    """Small-integer inputs: every partial sum exact, so any split gives the oracle's
    bits (ranges with no whole tile, only a tail, or nothing at all included)."""
    dtype = BF16
    M, N = 520, 392
    A, B = _layout_inputs(dtype, M, N, K, layout, 77 + K + layout, ints=True)
    want = orc.gemm(dtype, A, B, layout)
    for splits in (2, 4, 7, 64):
        say(f"quad split-K exact layout {layout} K={K} splits {splits}")
        got = _run_quad_split(dtype, A, B, layout, splits)
        assert np.array_equal(got, want), (K, splits)


def test_quad_split_repeat_launches_bitwise_identical(dev, orc):
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 1024, 768, 8192
    A, B = _inputs(BF16, M, N, K, 29)
    Ad, Bd = to_dev(A, BF16), to_dev(B, BF16)
    cfg = _quad_split(B_NK, 4)
    need = tgemm.workspace_size(M, N, cfg)
    ws = torch.empty((need // 4,), dtype=torch.int32, device="cuda")
    C0 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    tgemm.gemm_ex_ws(BF16, M, N, K, Ad, Bd, C0, ws, need, B_NK, cfg)
    torch.cuda.synchronize()
    ref = from_dev(C0)
    assert_parity(orc, BF16, K, ref, orc.gemm(BF16, A, B, B_NK), "quad split-K")
    say("quad split-K repeat launches")
    C = torch.empty_like(C0)
    for _ in range(10):
        tgemm.gemm_ex_ws(BF16, M, N, K, Ad, Bd, C, ws, need, B_NK, cfg)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(C), ref)


# ---------------------------------------------------------------------------------------
# Stream-K (TGEMM_KERNEL_QUAD_STREAMK): the tile rows filling whole waves as a plain quad
# product, the rest dealt in equal K-step ranges to 256 workgroups (at most two tile
# segments each), fp32 partials summed per tile in workgroup order.
# ---------------------------------------------------------------------------------------
def _quad_sk(layout):
    from tiled_dense_gemm_major_amd import tgemm
    return tgemm.Config(kernel=tgemm.KERNEL_QUAD_STREAMK, block_m=256, block_n=256,
                        block_k=64, waves_m=2, waves_n=2, stages=5, group_m=4, split_k=1,
                        mfma=16 if layout == B_NK else 32)


def _run_quad_sk(dtype, A, B, layout, guard=1024):
    from tiled_dense_gemm_major_amd import tgemm
    M, K = A.shape
    N = B.shape[0] if layout == B_NK else B.shape[1]
    cfg = _quad_sk(layout)
    need = tgemm.workspace_size(M, N, cfg)
    assert need == tgemm.STREAMK_WORKSPACE_BYTES
    ws = torch.full(((need + guard) // 4,), -1, dtype=torch.int32, device="cuda")
    C = torch.full((M, N), 0x7E00, dtype=torch.int16, device="cuda").view(tdtype(dtype))
    tgemm.gemm_ex_ws(dtype, M, N, K, to_dev(A, dtype), to_dev(B, dtype), C, ws, need, layout,
                     cfg)
    torch.cuda.synchronize()
    assert np.all(ws[need // 4:].cpu().numpy() == -1), "workspace written past its size"
    return from_dev(C)


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("layout", [B_NK, B_KN])
@pytest.mark.parametrize("shape", [
    (4500, 4000, 200),      # 18 x 16 tiles: 16 rows of whole waves, 2 rows by stream-K
    (600, 536, 1000),       # 9 tiles, fewer K steps than workgroups (empty ranges)
    (1000, 3000, 4104),     # 48 tiles of 65 steps: ranges across tile ends, a K tail
    (5000, 1512, 520)])     # 20 x 6 tiles
def test_quad_streamk_ragged(dev, orc, dtype, layout, shape):
    M, N, K = shape
    A, B = _layout_inputs(dtype, M, N, K, layout, 900 + M + N + K + layout)
    say(f"quad stream-K {dtype} layout {layout} {shape}")
    got = _run_quad_sk(dtype, A, B, layout)
    assert not np.any(got == 0x7E00)
    assert_parity(orc, dtype, K, got, orc.gemm(dtype, A, B, layout), f"stream-K {shape}")


@pytest.mark.parametrize("layout", [B_NK, B_KN])
@pytest.mark.parametrize("shape", [(1300, 2600, 4104), (4400, 4200, 136), (256, 66048, 64)])
def test_quad_streamk_exact_ints(dev, orc, layout, shape):
    """Small-integer inputs: the segments' partial sums are exact, so the stream-K result
    is the oracle's bit for bit (the last shape has more than 256 tiles in its one tile
    row, which runs as a plain quad product)."""
    M, N, K = shape
    A, B = _layout_inputs(BF16, M, N, K, layout, 31 + M + K + layout, ints=True)
    say(f"quad stream-K exact layout {layout} {shape}")
    assert np.array_equal(_run_quad_sk(BF16, A, B, layout), orc.gemm(BF16, A, B, layout))


def test_quad_streamk_repeat_launches_bitwise_identical(dev, orc):
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 4608, 4352, 2056            # 18 x 17 tiles: 15 whole-wave rows, 3 by stream-K
    A, B = _inputs(BF16, M, N, K, 37)
    Ad, Bd = to_dev(A, BF16), to_dev(B, BF16)
    cfg = _quad_sk(B_NK)
    need = tgemm.workspace_size(M, N, cfg)
    ws = torch.empty((need // 4,), dtype=torch.int32, device="cuda")
    C0 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    tgemm.gemm_ex_ws(BF16, M, N, K, Ad, Bd, C0, ws, need, B_NK, cfg)
    torch.cuda.synchronize()
    ref = from_dev(C0)
    assert_parity(orc, BF16, K, ref, orc.gemm(BF16, A, B, B_NK), "quad stream-K")
    say("quad stream-K repeat launches")
    C = torch.empty_like(C0)
    for _ in range(5):
        tgemm.gemm_ex_ws(BF16, M, N, K, Ad, Bd, C, ws, need, B_NK, cfg)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(C), ref)
