"""GPU parity: the HIP kernels, called through the C ABI, against the CPU oracle, element
by element, with |gpu - oracle| <= 1e-3*sqrt(K) + one output ulp of |oracle|; bit for bit
where every partial sum is exact."""
import numpy as np
import pytest

from tests.gpu_util import (assert_parity, assert_parity_full, from_dev, require_gpu, run,
                            sample_positions, say, tdtype, to_dev, torch)
from tiled_dense_gemm_major_amd.inputs import (BF16, B_KN, B_NK, F16, WORKLOADS, Stream,
                                               Workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _inputs(dtype, M, N, K, layout, seed, dist="uniform"):
    s = Stream(seed)
    A = s.matrix((M, K), dtype, dist)
    B = s.matrix((N, K) if layout == B_NK else (K, N), dtype, dist)
    return A, B


def _configs(dtype, layout):
    from tiled_dense_gemm_major_amd import tgemm
    return tgemm.list_configs(dtype, layout)


def _cfg_id(c):
    return (f"k{c.kernel}_{c.block_m}x{c.block_n}x{c.block_k}_w{c.waves_m}x{c.waves_n}"
            f"_s{c.stages}_m{c.mfma}")


# ---------------------------------------------------------------------------------------
# Every compiled configuration on ragged shapes spanning several tiles.
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("layout", [B_NK, B_KN])
def test_every_config_ragged(dev, orc, dtype, layout):
    M, N, K = 600, 536, 328          # ragged against 64/128/256 tiles; K tail of 8 past 64
    A, B = _inputs(dtype, M, N, K, layout, 100 + dtype + 2 * layout)
    want = orc.gemm(dtype, A, B, layout)
    for cfg in _configs(dtype, layout):
        say(f"config {_cfg_id(cfg)} dtype {dtype} layout {layout} {M}x{N}x{K}")
        got = run(dtype, A, B, layout, cfg)
        assert_parity(orc, dtype, K, got, want, _cfg_id(cfg))


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("layout", [B_NK, B_KN])
@pytest.mark.parametrize("shape", [(1, 8, 8), (8, 8, 16), (33, 40, 72), (257, 264, 1000),
                                   (64, 1024, 2048), (300, 8, 520), (1, 264, 1032),
                                   (50, 200, 4104), (100, 96, 1024), (128, 40, 3000)])
def test_table_choice_shapes(dev, orc, dtype, layout, shape):
    M, N, K = shape
    A, B = _inputs(dtype, M, N, K, layout, 7 + M + N + K)
    say(f"table choice {dtype} {layout} {shape}")
    got = run(dtype, A, B, layout)
    assert_parity(orc, dtype, K, got, orc.gemm(dtype, A, B, layout), str(shape))


# ---------------------------------------------------------------------------------------
# Exact arithmetic: small integers make every fp32 partial sum exact, so any summation
# order gives the oracle's bits.  Index-coded and one-hot inputs catch mapping bugs.
# ---------------------------------------------------------------------------------------
def _int_bits(dtype, arr):
    from tiled_dense_gemm_major_amd.inputs import round_to_bf16_bits, round_to_f16_bits
    f = round_to_f16_bits if dtype == F16 else round_to_bf16_bits
    return f(np.asarray(arr, dtype=np.float64))


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("layout", [B_NK, B_KN])
def test_exact_small_integers_bitwise(dev, orc, dtype, layout):
    rng = np.random.default_rng(17)
    M, N, K = 520, 392, 264
    A = _int_bits(dtype, rng.integers(-2, 3, (M, K)))
    Bn = _int_bits(dtype, rng.integers(-2, 3, (N, K)))
    B = Bn if layout == B_NK else np.ascontiguousarray(Bn.T)
    want = orc.gemm(dtype, A, B, layout)
    for cfg in _configs(dtype, layout):
        say(f"exact ints {_cfg_id(cfg)}")
        got = run(dtype, A, B, layout, cfg)
        assert np.array_equal(got, want), _cfg_id(cfg)


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_index_coded_and_one_hot_k(dev, orc, dtype):
    # A[m,k] = 1 only at k = K-1 (catches K-tail bugs); B[n,k] = n/8 at k = K-1, so
    # C[m,n] = n/8 exactly: column mapping is visible in every element.
    M, N, K = 300, 272, 200
    A = np.zeros((M, K)); A[:, K - 1] = 1.0
    B = np.zeros((N, K)); B[:, K - 1] = np.arange(N) / 8.0
    A, B = _int_bits(dtype, A), _int_bits(dtype, B)
    want = orc.gemm(dtype, A, B, B_NK)
    for cfg in _configs(dtype, B_NK):
        say(f"one-hot k {_cfg_id(cfg)}")
        assert np.array_equal(run(dtype, A, B, B_NK, cfg), want), _cfg_id(cfg)
    # row-coded: A[m, k] = (m % 64) / 8 at k = 0 only, B = 1 at k = 0: C[m, n] = (m%64)/8
    A = np.zeros((M, K)); A[:, 0] = (np.arange(M) % 64) / 8.0
    B = np.zeros((N, K)); B[:, 0] = 1.0
    A, B = _int_bits(dtype, A), _int_bits(dtype, B)
    want = orc.gemm(dtype, A, B, B_NK)
    for cfg in _configs(dtype, B_NK):
        say(f"row-coded {_cfg_id(cfg)}")
        assert np.array_equal(run(dtype, A, B, B_NK, cfg), want), _cfg_id(cfg)


# ---------------------------------------------------------------------------------------
# Degenerate and awkward arguments.
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_k_zero_writes_zeros(dev, orc, dtype):
    A = np.zeros((70, 0), dtype=np.uint16)
    B = np.zeros((0, 90), dtype=np.uint16)
    say("k = 0")
    got = run(dtype, A, B, B_KN)
    assert got.shape == (70, 90) and np.all(got == 0)


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("layout", [B_NK, B_KN])
@pytest.mark.parametrize("shape,offsets", [((77, 51, 37), (0, 0, 0)),   # K, N not x8
                                           ((128, 128, 128), (1, 0, 0)),  # A misaligned
                                           ((128, 128, 128), (0, 3, 0)),  # B misaligned
                                           ((128, 128, 128), (0, 0, 5)),  # C misaligned
                                           ((5, 3, 1), (0, 0, 0))])
def test_unaligned_and_odd_sizes(dev, orc, dtype, layout, shape, offsets):
    M, N, K = shape
    A, B = _inputs(dtype, M, N, K, layout, 55 + M)
    say(f"odd sizes {shape} offsets {offsets}")
    got = run(dtype, A, B, layout, a_offset=offsets[0], b_offset=offsets[1],
              c_offset=offsets[2])
    assert_parity(orc, dtype, K, got, orc.gemm(dtype, A, B, layout), str((shape, offsets)))


def test_does_not_write_outside_c(dev, orc):
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 200, 136, 96
    A, B = _inputs(BF16, M, N, K, B_NK, 3)
    guard = 4096
    buf = torch.full((guard + M * N + guard,), 0x1234, dtype=torch.int16, device="cuda")
    C = buf[guard:guard + M * N].view(torch.bfloat16).view(M, N)
    say("guard bands")
    tgemm.gemm_bf16(M, N, K, to_dev(A, BF16), to_dev(B, BF16), C)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:guard] == 0x1234) and np.all(host[guard + M * N:] == 0x1234)


def test_repeat_launches_bitwise_identical(dev, orc):
    """Stage-reuse races show up as rare differences between launches (the tutorial's
    corrupted-barrier lesson): the kernels have a fixed order and no atomics, so every
    launch must give the same bits, with no NaN."""
    from tiled_dense_gemm_major_amd import tgemm
    w = WORKLOADS["bf16_4096"]
    M, N, K = 2048, 2048, 4096
    A, B = _inputs(BF16, M, N, K, B_NK, 77)
    Ad, Bd = to_dev(A, BF16), to_dev(B, BF16)
    C0 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    tgemm.gemm_bf16(M, N, K, Ad, Bd, C0)
    ref = from_dev(C0)
    assert not np.any(np.isnan(ref.view(np.uint16).astype(np.uint32) << 16)
                      .view(np.float32))
    say(f"repeat launches {w.name}-like {M}x{N}x{K}")
    C = torch.empty_like(C0)
    for _ in range(30):
        tgemm.gemm_bf16(M, N, K, Ad, Bd, C)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(C), ref)


def test_stream_argument(dev, orc):
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 256, 256, 256
    A, B = _inputs(F16, M, N, K, B_NK, 9)
    s = torch.cuda.Stream()
    Ad, Bd = to_dev(A, F16), to_dev(B, F16)
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        tgemm.gemm_f16(M, N, K, Ad, Bd, C, stream=s)
    s.synchronize()
    assert_parity(orc, F16, K, from_dev(C), orc.gemm(F16, A, B, B_NK), "stream")


# ---------------------------------------------------------------------------------------
# The five workloads at their full sizes, in the configuration the table picks (the one
# the benchmark times), every element of C against the oracle (run over row blocks);
# the large ones get a quick sampled pass first so a gross failure shows at once.
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full_size(dev, orc, name):
    w = WORKLOADS[name]
    A, B = w.generate()
    say(f"workload {w.name}: {w.describe()}")
    got = run(w.dtype, A, B, w.b_layout)
    assert not np.any(got == 0x7E00)     # every element written
    if w.M * w.N * w.K > 2 ** 34:
        rows, cols = sample_positions(w.M, w.N, 3000, w.seed)
        want, _ = orc.gemm_entries(w.dtype, A, B, w.b_layout, rows, cols)
        assert_parity(orc, w.dtype, w.K, got[rows, cols], want, name + " sampled")
        say(f"workload {w.name}: sampled pass done, comparing all of C")
    worst = assert_parity_full(orc, w.dtype, A, B, w.b_layout, got, name)
    say(f"workload {w.name}: {w.M * w.N} elements, worst error {worst:.3f} of tolerance")


# ---------------------------------------------------------------------------------------
# Short K walks: fewer K tiles than pipeline slots (loads of tiles past the end must add
# nothing), and K tails inside the last tile, for every compiled configuration.
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("K", [8, 64, 72, 128, 200])
def test_every_config_short_k_exact(dev, orc, dtype, K):
    rng = np.random.default_rng(K)
    M, N = 264, 520
    A = _int_bits(dtype, rng.integers(-2, 3, (M, K)))
    B = _int_bits(dtype, rng.integers(-2, 3, (N, K)))
    want = orc.gemm(dtype, A, B, B_NK)
    for cfg in _configs(dtype, B_NK):
        say(f"short k {K} {_cfg_id(cfg)}")
        assert np.array_equal(run(dtype, A, B, B_NK, cfg), want), (K, _cfg_id(cfg))


# K walks of the quadrant kernel, bit for bit on exact inputs: the steps run as
# (K/64 mod 6) single steps and then groups of six with constant ring slots, a K tail is
# walked first, and the XCD-staggered walk wraps at the last whole tile.  Each K below
# picks one combination (whole tiles, tail, remainder steps, groups).
@pytest.mark.parametrize("layout", [B_NK, B_KN])
@pytest.mark.parametrize("K", [8, 136, 192, 384, 448, 456, 712, 776, 1000, 1536])
def test_quad_k_walk_exact(dev, orc, K, layout):
    from tiled_dense_gemm_major_amd import tgemm
    dtype = BF16
    rng = np.random.default_rng(500 + K)
    M, N = 512, 768          # 2 x 3 tiles, so the eight XCD staggers differ
    A = _int_bits(dtype, rng.integers(-2, 3, (M, K)))
    Bn = _int_bits(dtype, rng.integers(-2, 3, (N, K)))
    B = Bn if layout == B_NK else np.ascontiguousarray(Bn.T)
    want = orc.gemm(dtype, A, B, layout)
    nk = -(-K // 64)
    cfgs = [c for c in _configs(dtype, layout) if c.kernel == tgemm.KERNEL_QUAD]
    assert cfgs
    for cfg in cfgs:
        say(f"quad k walk K={K} layout {layout} (tiles {nk}, remainder {nk % 6}, "
            f"tail {K % 64}) {_cfg_id(cfg)}")
        assert np.array_equal(run(dtype, A, B, layout, cfg), want), (K, _cfg_id(cfg))


# K walks of the direct kernel, bit for bit on exact inputs: its four waves take a
# quarter each of the 16-wide k blocks, in batches of eight (four for 128-row tiles), so
# these K give waves with no block, one batch, a partial batch, odd and even numbers of
# batches, and a final block with only its first half inside K.
@pytest.mark.parametrize("K", [8, 16, 40, 72, 136, 512, 520, 1000, 1032, 2056])
def test_direct_k_walk_exact(dev, orc, K):
    from tiled_dense_gemm_major_amd import tgemm
    dtype = F16
    rng = np.random.default_rng(900 + K)
    M, N = 200, 264          # 7 x 9 tiles of 32, ragged in both
    A = _int_bits(dtype, rng.integers(-2, 3, (M, K)))
    B = _int_bits(dtype, rng.integers(-2, 3, (N, K)))
    want = orc.gemm(dtype, A, B, B_NK)
    cfgs = [c for c in _configs(dtype, B_NK) if c.kernel == tgemm.KERNEL_DIRECT]
    assert cfgs
    for cfg in cfgs:
        say(f"direct k walk K={K} (blocks {-(-K // 16)}) {_cfg_id(cfg)}")
        assert np.array_equal(run(dtype, A, B, B_NK, cfg), want), (K, _cfg_id(cfg))


# K walks of the skinny kernel, bit for bit on exact inputs: each of its 8 waves walks a
# contiguous range of 64- or 128-wide chunks, starting at a chunk set by the workgroup's
# index on its XCD, so with 33 column blocks and 1-6 chunks per wave the ragged last
# chunk is reached first, last and in between.  The row counts leave 1 to 7 of a row block's
# 8-row A loads past M (not issued: their LDS rows are zeroed once), including a last
# row block of 36 rows (M = 100).  With B [K,N] the 33 column blocks also leave a ragged
# last group of the pairing of column blocks onto XCDs.
@pytest.mark.parametrize("layout", [B_NK, B_KN])
@pytest.mark.parametrize("K", [1000, 1544, 2568, 3080])
@pytest.mark.parametrize("M", [1, 9, 16, 64, 100])
def test_skinny_k_walk_exact(dev, orc, M, K, layout):
    from tiled_dense_gemm_major_amd import tgemm
    dtype = BF16
    rng = np.random.default_rng(700 + K + M)
    N = 1056
    A = _int_bits(dtype, rng.integers(-2, 3, (M, K)))
    B = _int_bits(dtype, rng.integers(-2, 3, (N, K)))
    want = orc.gemm(dtype, A, B, B_NK)
    Bl = B if layout == B_NK else np.ascontiguousarray(B.T)
    cfgs = [c for c in _configs(dtype, layout) if c.kernel == tgemm.KERNEL_SKINNY]
    assert cfgs
    for cfg in cfgs:
        say(f"skinny k walk M={M} K={K} layout {layout} (chunks {-(-K // cfg.block_k)}, "
            f"tail {K % cfg.block_k}) {_cfg_id(cfg)}")
        assert np.array_equal(run(dtype, A, Bl, layout, cfg), want), (M, K, _cfg_id(cfg))


@pytest.mark.parametrize("layout", [B_NK, B_KN])
def test_quad_repeat_launches_bitwise_identical(dev, orc, layout):
    """Many workgroups per compute unit through the five-slot ring: a stage reused too
    early shows up as launch-to-launch differences."""
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 2048, 2304, 1536
    A, B = _inputs(BF16, M, N, K, layout, 91)
    Ad, Bd = to_dev(A, BF16), to_dev(B, BF16)
    for cfg in [c for c in _configs(BF16, layout) if c.kernel == tgemm.KERNEL_QUAD]:
        say(f"quad repeat launches layout {layout} {_cfg_id(cfg)} mfma {cfg.mfma}")
        C0 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        tgemm.gemm_ex(BF16, M, N, K, Ad, Bd, C0, layout, cfg)
        torch.cuda.synchronize()
        ref = from_dev(C0)
        assert_parity_full(orc, BF16, A, B, layout, ref, "quad")
        C = torch.empty_like(C0)
        for _ in range(20):
            tgemm.gemm_ex(BF16, M, N, K, Ad, Bd, C, layout, cfg)
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(C), ref)


# ---------------------------------------------------------------------------------------
# B [K,N] through the quad kernel: column- and row-coded exact inputs (every element of C
# names the column or row it came from, so a wrong swizzle or transposing-read lane shows
# as a wrong value), padded leading dimensions below and above the 256 the instruction-
# offset loads need, and the ragged workload and a 4096^3 product at full size.
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_quad_kn_coded_exact(dev, orc, dtype):
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 520, 776, 200
    cfgs = [c for c in _configs(dtype, B_KN) if c.kernel == tgemm.KERNEL_QUAD]
    assert cfgs
    # column-coded: B[k, n] = (n % 128) / 8 + 1 at k = K - 1 (else 0), A[:, K - 1] = 1
    A = np.zeros((M, K)); A[:, K - 1] = 1.0
    B = np.zeros((K, N)); B[K - 1, :] = (np.arange(N) % 128) / 8.0 + 1.0
    A, B = _int_bits(dtype, A), _int_bits(dtype, B)
    want = orc.gemm(dtype, A, B, B_KN)
    for cfg in cfgs:
        say(f"quad [K,N] column-coded {_cfg_id(cfg)}")
        assert np.array_equal(run(dtype, A, B, B_KN, cfg), want), _cfg_id(cfg)
    # k-coded: B[k, n] = (k % 64) / 8 for one column block, A = 1: C[m, n] = the sum
    # over k, exact; every k row of every slot contributes its own value
    A = np.ones((M, K))
    B = np.zeros((K, N)); B[:, :] = ((np.arange(K) % 64) / 8.0)[:, None]
    B[:, 300:] = ((np.arange(K) % 16) / 4.0)[:, None] * ((np.arange(N - 300) % 3) - 1)
    A, B = _int_bits(dtype, A), _int_bits(dtype, B)
    want = orc.gemm(dtype, A, B, B_KN)
    for cfg in cfgs:
        say(f"quad [K,N] k-coded {_cfg_id(cfg)}")
        assert np.array_equal(run(dtype, A, B, B_KN, cfg), want), _cfg_id(cfg)


@pytest.mark.parametrize("name", ["f16_4000x3000x1000_kn"])
def test_quad_kn_ragged_workload_full(dev, orc, name):
    """The ragged [K,N] workload (edge tiles, K tail of 40) through each quad
    configuration, every element against the oracle."""
    from tiled_dense_gemm_major_amd import tgemm
    w = WORKLOADS[name]
    A, B = w.generate()
    want = orc.gemm(w.dtype, A, B, w.b_layout)
    for cfg in [c for c in _configs(w.dtype, B_KN) if c.kernel == tgemm.KERNEL_QUAD]:
        say(f"quad [K,N] {w.describe()} {_cfg_id(cfg)}")
        got = run(w.dtype, A, B, w.b_layout, cfg)
        assert_parity(orc, w.dtype, w.K, got, want, _cfg_id(cfg))


def test_quad_kn_4096_full(dev, orc):
    from tiled_dense_gemm_major_amd import tgemm
    M = N = K = 4096
    A, B = _inputs(BF16, M, N, K, B_KN, 4096)
    want = orc.gemm(BF16, A, B, B_KN)
    for cfg in [c for c in _configs(BF16, B_KN) if c.kernel == tgemm.KERNEL_QUAD]:
        say(f"quad [K,N] 4096^3 {_cfg_id(cfg)}")
        assert_parity(orc, BF16, K, run(BF16, A, B, B_KN, cfg), want, _cfg_id(cfg))


# ---------------------------------------------------------------------------------------
# Non-finite results: NaN and infinite inputs, and sums past the output format's range.
# The acceptance rule fails every non-finite GPU value, so these are checked by class:
# where the oracle's result is NaN the GPU's must be NaN, where it is +-inf the GPU's must
# be the same infinity, and every other element meets the rule.  Finite magnitudes stay
# small enough that no fp32 partial sum overflows where the fp64 sum would not.
# ---------------------------------------------------------------------------------------
def _special_inputs(dtype, M, N, K, layout, seed):
    from tiled_dense_gemm_major_amd.inputs import round_to_bf16_bits, round_to_f16_bits
    enc = round_to_f16_bits if dtype == F16 else round_to_bf16_bits
    nan, pinf, ninf = (0x7E00, 0x7C00, 0xFC00) if dtype == F16 else (0x7FC0, 0x7F80, 0xFF80)
    rng = np.random.default_rng(seed)
    a = rng.uniform(-1, 1, (M, K))
    b = rng.uniform(-1, 1, (N, K))
    b[:, 9] = np.abs(b[:, 9]) + 0.5                    # for row 7's +inf at k = 9
    b[11, 9] = 0.0                                     # ... inf x 0: NaN in column 11
    a[:, 2] = np.abs(a[:, 2]) + 0.25                   # for column 17's -inf at k = 2
    a[7, :] = 0.0
    # rows 20-23 x columns 30-33 past the largest finite value, through one k only: a
    # product of two large values there, every other term of those sums (and every term
    # elsewhere) small, so no fp32 partial sum can overflow where the fp64 sum does not
    big = 300.0 if dtype == F16 else 3.0e37
    b[:, 40] = rng.uniform(-1e-3, 1e-3, N)
    a[20:24, 40] = big
    b[30:34, 40] = big
    A = enc(a)
    Bn = enc(b)
    A[3, 5] = nan                                      # row 3 of C: NaN
    A[7, 9] = pinf                                     # row 7: +inf, NaN at column 11
    Bn[17, 2] = ninf                                   # column 17: -inf (row 7: 0 x -inf)
    B = Bn if layout == B_NK else np.ascontiguousarray(Bn.T)
    return A, B


def _assert_same_class(orc, dtype, K, got, want, what):
    g = orc.decode(dtype, got).ravel()
    w = orc.decode(dtype, want).ravel()
    assert np.array_equal(np.isnan(g), np.isnan(w)), f"{what}: NaN positions differ"
    inf = np.isinf(w)
    assert np.array_equal(np.isinf(g), inf), f"{what}: infinite positions differ"
    assert np.array_equal(np.sign(g[inf]), np.sign(w[inf])), f"{what}: infinity signs differ"
    fin = np.isfinite(w)
    res = orc.compare(dtype, K, got.ravel()[fin], want.ravel()[fin])
    assert res["n_fail"] == 0, f"{what}: {res}"
    return int(np.isnan(w).sum()), int(inf.sum())


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("layout", [B_NK, B_KN])
def test_every_config_non_finite(dev, orc, dtype, layout):
    M, N, K = 200, 264, 72
    A, B = _special_inputs(dtype, M, N, K, layout, 61 + dtype + 2 * layout)
    want = orc.gemm(dtype, A, B, layout)
    n_nan, n_inf = _assert_same_class(orc, dtype, K, want, want, "oracle")
    assert n_nan > 0 and n_inf > 0
    for cfg in _configs(dtype, layout):
        say(f"non-finite {_cfg_id(cfg)} dtype {dtype} layout {layout}")
        got = run(dtype, A, B, layout, cfg)
        _assert_same_class(orc, dtype, K, got, want, _cfg_id(cfg))


# ---------------------------------------------------------------------------------------
# Skinny kernels with A [M,K] and B [N,K] meeting the fast rules while C does not (odd N,
# an odd leading dimension, a C base off 16 bytes): C is stored element by element where
# its rows are unaligned, and nothing outside C's rows may change.
# ---------------------------------------------------------------------------------------
def _run_strided_c(dtype, A_bits, B_bits, ldc, c_offset, config=None, guard=64,
                   fill=0x7E00):
    from tiled_dense_gemm_major_amd import tgemm
    M, K = A_bits.shape
    N = B_bits.shape[0]
    A, B = to_dev(A_bits, dtype), to_dev(B_bits, dtype)
    total = c_offset + (M - 1) * ldc + N + guard
    buf = torch.full((total,), fill, dtype=torch.int16, device="cuda")
    C = buf.view(tdtype(dtype))[c_offset:]
    tgemm.gemm_strided(dtype, M, N, K, A, K, tgemm.A_MK, B, K, tgemm.B_NK, C, ldc, config)
    torch.cuda.synchronize()
    host = buf.cpu().numpy().view(np.uint16)
    outside = np.ones(total, dtype=bool)
    rows = []
    for r in range(M):
        lo = c_offset + r * ldc
        rows.append(host[lo:lo + N].copy())
        outside[lo:lo + N] = False
    assert np.all(host[outside] == fill), "an element outside C's rows changed"
    return np.stack(rows)


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("M", [1, 9, 32, 64])
@pytest.mark.parametrize("N,ldc,c_offset", [(257, 257, 0), (1031, 1031, 1), (1056, 1059, 0),
                                            (1056, 1056, 3), (1063, 1070, 2)])
def test_skinny_unaligned_c_exact(dev, orc, dtype, M, N, ldc, c_offset):
    from tiled_dense_gemm_major_amd import tgemm
    K = 1032                              # a multiple of 8, with a chunk tail
    rng = np.random.default_rng(900 + M + N + ldc + c_offset)
    A = _int_bits(dtype, rng.integers(-2, 3, (M, K)))
    B = _int_bits(dtype, rng.integers(-2, 3, (N, K)))
    want = orc.gemm(dtype, A, B, B_NK)
    assert tgemm.query_config(dtype, M, N, K, B_NK, tgemm.ALIGN_OPERANDS).kernel == \
        tgemm.KERNEL_SKINNY
    say(f"skinny unaligned C M={M} N={N} ldc={ldc} offset={c_offset} table choice")
    assert np.array_equal(_run_strided_c(dtype, A, B, ldc, c_offset), want)
    for cfg in [c for c in _configs(dtype, B_NK) if c.kernel == tgemm.KERNEL_SKINNY]:
        say(f"skinny unaligned C M={M} N={N} ldc={ldc} offset={c_offset} {_cfg_id(cfg)}")
        assert np.array_equal(_run_strided_c(dtype, A, B, ldc, c_offset, cfg), want), \
            _cfg_id(cfg)


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_skinny_odd_vocabulary_full(dev, orc, dtype):
    """A decode step's output projection over an odd vocabulary (8 x 50257 x 4096, packed,
    so every C row but the first is unaligned): the packed entry point takes the skinny
    kernel, every element against the oracle."""
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = 8, 50257, 4096
    assert tgemm.query_config_packed(dtype, M, N, K).kernel == tgemm.KERNEL_SKINNY
    s = Stream(61)
    A = s.matrix((M, K), dtype, "normal")
    B = s.matrix((N, K), dtype, "normal")
    say(f"odd vocabulary {M}x{N}x{K} dtype {dtype}")
    Ad, Bd = to_dev(A, dtype), to_dev(B, dtype)
    C = torch.full((M, N), 0x7E00, dtype=torch.int16, device="cuda").view(tdtype(dtype))
    (tgemm.gemm_f16 if dtype == F16 else tgemm.gemm_bf16)(M, N, K, Ad, Bd, C)
    torch.cuda.synchronize()
    assert_parity_full(orc, dtype, A, B, B_NK, from_dev(C), "odd vocabulary")


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("shape,layout,kernel", [
    ((24, 12288, 1024), B_NK, "skinny64"), ((80, 12288, 1024), B_NK, "dma"),
    ((72, 20480, 1024), B_NK, "tiled"),
    ((16, 40960, 1024), B_NK, "quad"), ((8, 40960, 1024), B_NK, "skinny"),
    ((40, 28672, 1024), B_KN, "quad"), ((8, 28672, 1024), B_KN, "skinny"),
    ((136, 12296, 1032), B_KN, "quad"), ((100, 12288, 1024), B_KN, "quad")])
def test_wide_n_table_choices(dev, orc, dtype, shape, layout, kernel):
    """Products past the table's widest N take the rule's choice through the default path;
    every element against the oracle."""
    from tiled_dense_gemm_major_amd import tgemm
    M, N, K = shape
    c = tgemm.query_config(dtype, M, N, K, layout)
    want_kernel = {"skinny64": tgemm.KERNEL_SKINNY, "skinny": tgemm.KERNEL_SKINNY,
                   "tiled": tgemm.KERNEL_TILED, "quad": tgemm.KERNEL_QUAD,
                   "dma": tgemm.KERNEL_DMA}[kernel]
    assert c.kernel == want_kernel, c
    if kernel == "skinny64":
        assert c.block_n == 64
    if kernel == "tiled":
        assert (c.block_m, c.block_n) == (128, 128)
    A, B = _inputs(dtype, M, N, K, layout, 800 + M)
    say(f"wide N {shape} layout {layout} dtype {dtype} -> {_cfg_id(c)}")
    got = run(dtype, A, B, layout)
    assert_parity(orc, dtype, K, got, orc.gemm(dtype, A, B, layout), str(shape))
