"""GPU parity of the general product (gemm_strided): A stored [M,K] or [K,M], B stored
[N,K] or [K,N], each operand and C with a leading dimension larger than its row.  The
padding between rows holds NaN patterns, so a kernel that read it would poison C, and C's
own padding must come back untouched.  The oracle sees the same logical operands."""
import numpy as np
import pytest

from tests.gpu_util import assert_parity, from_dev, require_gpu, say, tdtype, torch
from tiled_dense_gemm_major_amd.inputs import BF16, B_KN, B_NK, F16, Stream

pytestmark = pytest.mark.gpu

A_MK, A_KM = 0, 1
POISON = 0x7E00          # a NaN in both fp16 and bf16 (and the C sentinel)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _store(logical, transposed, pad):
    """The storage of a logical [R, K] operand: [R, K + pad] (row-major, K contiguous) or
    [K, R + pad] (transposed), padding filled with POISON.  Returns (storage, ld)."""
    R, K = logical.shape
    if transposed:
        st = np.full((K, R + pad), POISON, dtype=np.uint16)
        st[:, :R] = logical.T
        return st, R + pad
    st = np.full((R, K + pad), POISON, dtype=np.uint16)
    st[:, :K] = logical
    return st, K + pad


def _shifted(st, off):
    """A device copy of `st` starting `off` elements into its allocation (the elements
    before it hold POISON): a base address off * 2 bytes past 16-byte alignment."""
    flat = torch.full((off + st.size,), POISON, dtype=torch.int16, device="cuda")
    flat[off:] = torch.from_numpy(st.reshape(-1).view(np.int16)).cuda()
    return flat, flat[off:]


def run_strided(dtype, A, Bn, a_layout, b_layout, pads=(8, 16, 24), config=None,
                offsets=(0, 0, 0)):
    """C = A x Bn^T (logical A [M,K], Bn [N,K]) through gemm_strided with the given
    storages, each base address `offsets` elements past an aligned allocation; returns
    C's bits and checks that neither its padding nor the elements before it were
    written."""
    from tiled_dense_gemm_major_amd import tgemm
    M, K = A.shape
    N = Bn.shape[0]
    a_st, lda = _store(A, a_layout == A_KM, pads[0])
    b_st, ldb = _store(Bn, b_layout == B_KN, pads[1])
    ldc = N + pads[2]
    _, Ad = _shifted(a_st, offsets[0])
    _, Bd = _shifted(b_st, offsets[1])
    c_all, Cd = _shifted(np.full((max(M, 1), ldc), POISON, dtype=np.uint16), offsets[2])
    tgemm.gemm_strided(dtype, M, N, K, Ad.view(tdtype(dtype)), lda, a_layout,
                       Bd.view(tdtype(dtype)), ldb, b_layout, Cd.view(tdtype(dtype)), ldc,
                       config)
    torch.cuda.synchronize()
    host = from_dev(c_all)
    assert np.all(host[:offsets[2]] == POISON), "elements before C were written"
    c = host[offsets[2]:].reshape(max(M, 1), ldc)
    assert np.all(c[:, N:] == POISON), "C padding was written"
    return c[:M, :N]


def _inputs(dtype, M, N, K, seed):
    s = Stream(seed)
    return s.matrix((M, K), dtype, "uniform"), s.matrix((N, K), dtype, "uniform")


def _int_bits(dtype, arr):
    from tiled_dense_gemm_major_amd.inputs import round_to_bf16_bits, round_to_f16_bits
    f = round_to_f16_bits if dtype == F16 else round_to_bf16_bits
    return f(np.asarray(arr, dtype=np.float64))


LAYOUTS = [(A_MK, B_NK), (A_MK, B_KN), (A_KM, B_NK), (A_KM, B_KN)]


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("a_layout,b_layout", LAYOUTS)
def test_strided_every_config(dev, orc, dtype, a_layout, b_layout):
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 600, 536, 328         # ragged against every tile; multiples of 8
    A, Bn = _inputs(dtype, M, N, K, 300 + 4 * dtype + 2 * a_layout + b_layout)
    want = orc.gemm(dtype, A, Bn, B_NK)
    for cfg in tgemm.list_configs(dtype, b_layout, a_layout):
        if tgemm.workspace_size(M, N, cfg):
            continue        # split-K needs a lent workspace: gemm_ex_ws only
        say(f"strided {dtype} A{a_layout} B{b_layout} {cfg.as_dict()}")
        got = run_strided(dtype, A, Bn, a_layout, b_layout, config=cfg)
        assert_parity(orc, dtype, K, got, want, str(cfg.as_dict()))


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("a_layout,b_layout", LAYOUTS)
def test_strided_exact_ints_bitwise(dev, orc, dtype, a_layout, b_layout):
    from tiled_dense_gemm_major_amd import tgemm
    rng = np.random.default_rng(23 + a_layout + 2 * b_layout)
    M, N, K = 520, 392, 264
    A = _int_bits(dtype, rng.integers(-2, 3, (M, K)))
    Bn = _int_bits(dtype, rng.integers(-2, 3, (N, K)))
    want = orc.gemm(dtype, A, Bn, B_NK)
    for cfg in tgemm.list_configs(dtype, b_layout, a_layout):
        if tgemm.workspace_size(M, N, cfg):
            continue        # split-K needs a lent workspace: gemm_ex_ws only
        say(f"strided exact {dtype} A{a_layout} B{b_layout} {cfg.as_dict()}")
        got = run_strided(dtype, A, Bn, a_layout, b_layout, pads=(16, 8, 8), config=cfg)
        assert np.array_equal(got, want), str(cfg.as_dict())


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("a_layout,b_layout", LAYOUTS)
@pytest.mark.parametrize("shape,pads", [((77, 51, 37), (3, 5, 7)),      # nothing x8
                                        ((128, 128, 128), (1, 0, 0)),   # lda odd
                                        ((128, 128, 128), (0, 0, 3)),   # ldc odd
                                        ((100, 64, 64), (0, 0, 0)),     # M % 8 != 0
                                        ((1, 1, 1), (0, 0, 0))])
def test_strided_table_choice_any_alignment(dev, orc, dtype, a_layout, b_layout, shape,
                                            pads):
    M, N, K = shape
    A, Bn = _inputs(dtype, M, N, K, 77 + M + sum(pads))
    say(f"strided table {dtype} A{a_layout} B{b_layout} {shape} pads {pads}")
    got = run_strided(dtype, A, Bn, a_layout, b_layout, pads=pads)
    assert_parity(orc, dtype, K, got, orc.gemm(dtype, A, Bn, B_NK), str((shape, pads)))


# The masked tiled kernel (TGEMM_KERNEL_MASKED): every configuration of each storage pair
# on operands with no alignment beyond 2 bytes -- odd sizes (K tails of 1-7 elements, M
# and N not multiples of 8), odd leading dimensions and base addresses an odd number of
# elements into their allocations.
MASKED_CASES = [((77, 51, 37), (3, 5, 7), (0, 0, 0)),
                ((613, 541, 203), (1, 3, 5), (1, 0, 3)),     # several tiles, K tail of 3
                ((301, 262, 130), (0, 0, 0), (1, 1, 1)),     # packed rows, odd bases
                ((130, 70, 7), (2, 1, 1), (3, 7, 1)),        # K shorter than one chunk
                ((1, 1, 1), (0, 0, 0), (1, 1, 1))]


def _masked_configs(dtype, a_layout, b_layout):
    from tiled_dense_gemm_major_amd import tgemm
    cfgs = [c for c in tgemm.list_configs(dtype, b_layout, a_layout)
            if c.kernel == tgemm.KERNEL_MASKED]
    assert len(cfgs) >= 2
    return cfgs


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("a_layout,b_layout", LAYOUTS)
def test_masked_every_config_unaligned(dev, orc, dtype, a_layout, b_layout):
    for (M, N, K), pads, offs in MASKED_CASES:
        A, Bn = _inputs(dtype, M, N, K, 1500 + M + K + 4 * a_layout + b_layout)
        want = orc.gemm(dtype, A, Bn, B_NK)
        for cfg in _masked_configs(dtype, a_layout, b_layout):
            say(f"masked {dtype} A{a_layout} B{b_layout} {M}x{N}x{K} pads {pads} "
                f"offsets {offs} {cfg.as_dict()}")
            got = run_strided(dtype, A, Bn, a_layout, b_layout, pads=pads, config=cfg,
                              offsets=offs)
            assert_parity(orc, dtype, K, got, want, str(((M, N, K), pads, offs)))


@pytest.mark.parametrize("a_layout,b_layout", LAYOUTS)
def test_masked_exact_ints_bitwise(dev, orc, a_layout, b_layout):
    """Small integers (every partial sum exact) through the masked kernel: the element
    masks at the K tail and the M / N edges, bit for bit."""
    for (M, N, K), pads, offs in [((523, 389, 267), (1, 1, 1), (1, 1, 1)),
                                  ((200, 133, 64), (5, 0, 3), (0, 3, 0))]:
        rng = np.random.default_rng(1700 + M + a_layout + 2 * b_layout)
        A = _int_bits(BF16, rng.integers(-2, 3, (M, K)))
        Bn = _int_bits(BF16, rng.integers(-2, 3, (N, K)))
        want = orc.gemm(BF16, A, Bn, B_NK)
        for cfg in _masked_configs(BF16, a_layout, b_layout):
            say(f"masked exact A{a_layout} B{b_layout} {M}x{N}x{K} {cfg.as_dict()}")
            got = run_strided(BF16, A, Bn, a_layout, b_layout, pads=pads, config=cfg,
                              offsets=offs)
            assert np.array_equal(got, want), ((M, N, K), pads, offs)


@pytest.mark.parametrize("a_layout,b_layout", LAYOUTS)
def test_strided_large_table_choice(dev, orc, a_layout, b_layout):
    """The large-tile kernels (every quad configuration of the storage pair, and the
    first ping-pong one) on padded rows, every element against the oracle."""
    from tiled_dense_gemm_major_amd import tgemm
    dtype = BF16
    M, N, K = 3584, 4096, 1000
    listed = tgemm.list_configs(dtype, b_layout, a_layout)
    cfgs = [c for c in listed if c.kernel == tgemm.KERNEL_QUAD]
    cfgs += [c for c in listed if c.kernel == tgemm.KERNEL_PINGPONG][:1]
    assert len(cfgs) >= 2
    A, Bn = _inputs(dtype, M, N, K, 900 + a_layout + 2 * b_layout)
    want = orc.gemm(dtype, A, Bn, B_NK)
    for cfg in cfgs + [None]:             # None: the library's own choice
        say(f"strided large A{a_layout} B{b_layout} {M}x{N}x{K} "
            f"{cfg.as_dict() if cfg is not None else 'table choice'}")
        got = run_strided(dtype, A, Bn, a_layout, b_layout, pads=(64, 8, 256), config=cfg)
        assert_parity(orc, dtype, K, got, want, "large")


def test_strided_packed_matches_gemm_ex(dev, orc):
    """With leading dimensions equal to the row lengths, gemm_strided runs the packed
    product: both match the oracle, and each other bit for bit (same table choice)."""
    from tests.gpu_util import run
    A, Bn = _inputs(BF16, 300, 264, 200, 5)
    got = run_strided(BF16, A, Bn, A_MK, B_NK, pads=(0, 0, 0))
    assert_parity(orc, BF16, 200, got, orc.gemm(BF16, A, Bn, B_NK), "strided packed")
    assert np.array_equal(got, run(BF16, A, Bn, B_NK))


@pytest.mark.parametrize("pads", [(8, 8, 0), (0, 64, 8), (64, 0, 0)])
def test_strided_quad_kn_leading_dims(dev, orc, pads):
    """The quad kernel for B [K,N] with padded rows: N = 200 gives ldb 208-264, below and
    above the 256 that its instruction-offset loads need."""
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 300, 200, 328
    A, Bn = _inputs(BF16, M, N, K, 1200 + sum(pads))
    for cfg in [c for c in tgemm.list_configs(BF16, B_KN, A_MK)
                if c.kernel == tgemm.KERNEL_QUAD]:
        say(f"strided quad [K,N] pads {pads} {cfg.as_dict()}")
        got = run_strided(BF16, A, Bn, A_MK, B_KN, pads=pads, config=cfg)
        assert_parity(orc, BF16, K, got, orc.gemm(BF16, A, Bn, B_NK), str(pads))


@pytest.mark.parametrize("b_layout", [B_NK, B_KN])
@pytest.mark.parametrize("K", [8, 200, 456, 1000])
def test_strided_quad_km_k_walk_exact(dev, orc, b_layout, K):
    """The quad kernel for A [K,M] on small-integer inputs (every partial sum exact): the
    K tail (rows of the A slot past K), the six-step groups and row blocks past M, bit
    for bit.  M = 200 with lda = 208 takes the M0-walk loads (lda < 256); M = 520 with
    lda = 776 the instruction-offset ones."""
    from tiled_dense_gemm_major_amd import tgemm
    N = 776
    cfgs = [c for c in tgemm.list_configs(BF16, b_layout, A_KM)
            if c.kernel == tgemm.KERNEL_QUAD]
    assert cfgs
    for M, pads in [(200, (8, 0, 8)), (520, (256, 8, 0))]:
        rng = np.random.default_rng(1300 + K + b_layout + M)
        A = _int_bits(BF16, rng.integers(-2, 3, (M, K)))
        Bn = _int_bits(BF16, rng.integers(-2, 3, (N, K)))
        want = orc.gemm(BF16, A, Bn, B_NK)
        for cfg in cfgs:
            say(f"quad [K,M] M={M} K={K} B{b_layout} pads {pads} {cfg.as_dict()}")
            got = run_strided(BF16, A, Bn, A_KM, b_layout, pads=pads, config=cfg)
            assert np.array_equal(got, want), (M, K, pads)
