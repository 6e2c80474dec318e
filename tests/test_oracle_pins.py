"""Pins for the CPU oracle against what the pages and the mathematics fix, independent of
the oracle's own code: library routines (numpy, torch, Python fractions), exact integer
arithmetic, closed forms, invariants and the values printed on the pages."""
from fractions import Fraction

import numpy as np
import pytest

from tests.conftest import golden
from tiled_dense_gemm_major_amd.inputs import (BF16, B_KN, B_NK, F16, WORKLOADS, Stream,
                                               round_to_bf16_bits, splitmix64)

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


# --------------------------------------------------------------------------------------
# Codec: decode and the single rounding, against library routines and exact rationals.
# --------------------------------------------------------------------------------------
def test_decode_f16_exhaustive(orc):
    got = orc.decode(F16, ALL16)
    want = ALL16.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_bf16_exhaustive(orc):
    torch = pytest.importorskip("torch")
    got = orc.decode(BF16, ALL16)
    want = torch.from_numpy(ALL16.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def _f16_probe_values(rng):
    fin = ALL16.view(np.float16)
    fin = np.sort(np.unique(fin[np.isfinite(fin)].astype(np.float64)))
    mids = (fin[:-1] + fin[1:]) / 2          # exact in fp64
    up = np.nextafter(mids, np.inf)
    dn = np.nextafter(mids, -np.inf)
    rand = rng.standard_normal(1_000_000) * np.exp2(rng.integers(-30, 18, 1_000_000))
    edge = np.array([65504.0, 65519.999, 65520.0, 65536.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                     2.0 ** -25 * 1.0000001, 2.0 ** -26, 1e-300, 0.0, -0.0, np.inf, -np.inf])
    return np.concatenate([fin, mids, up, dn, rand, edge, -edge])


def test_encode_f16_matches_numpy(orc):
    rng = np.random.default_rng(123)
    x = _f16_probe_values(rng)
    got = orc.encode(F16, x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    nanbits = orc.encode(F16, np.array([np.nan]))
    assert np.isnan(nanbits.view(np.float16)[0])


def _exact_round(v, frac_bits: int, emin: int, emax: int):
    """Correct rounding (nearest, ties to even) of an exact rational to a binary format
    with ``frac_bits`` fraction bits and normal exponents [emin, emax]; None on overflow."""
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    sgn = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = Fraction(2) ** (max(e, emin) - frac_bits)
    n = a / q
    r = n.numerator // n.denominator
    rem = n - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    res = r * q
    if res >= Fraction(2) ** (emax + 1):
        return None
    return sgn * res


def _bf16_bits_to_fraction(b: int):
    sign = -1 if b >> 15 else 1
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    if e == 0:
        return sign * Fraction(f) * Fraction(2) ** -133
    if e == 255:
        return None
    return sign * Fraction(f | 0x80) * Fraction(2) ** (e - 134)


def test_encode_bf16_exact_rationals(orc):
    rng = np.random.default_rng(7)
    bf = ALL16[((ALL16 >> 7) & 0xFF) != 0xFF]
    vals = orc.decode(BF16, bf)
    vals = np.unique(vals[vals >= 0])
    mids = (vals[:-1] + vals[1:]) / 2
    pick = rng.choice(mids.size, 3000, replace=False)
    xs = np.concatenate([mids[pick], np.nextafter(mids[pick], np.inf),
                         np.nextafter(mids[pick], -np.inf),
                         rng.standard_normal(3000) * np.exp2(rng.integers(-140, 128, 3000)),
                         [3.3895313892515355e38, 3.4e38, 2.0 ** -133, 2.0 ** -134,
                          2.0 ** -134 * 1.5, 1e-45]])
    xs = np.concatenate([xs, -xs])
    got = orc.encode(BF16, xs)
    for x, g in zip(xs.tolist(), got.tolist()):
        want = _exact_round(x, 7, -126, 127)
        if want is None:
            assert (g & 0x7FFF) == 0x7F80, x
        else:
            assert _bf16_bits_to_fraction(g) == want, (x, hex(g))


def test_encode_bf16_matches_round_to_odd(orc):
    """Cross-check with a published route: fp64 -> fp32 with round-to-odd, then
    nearest-even to bf16 (Boldo & Melquiond, 'Emulation of FMA and correctly rounded sums:
    proved algorithms using rounding to odd', IEEE TC 2008): exact when the middle format
    has at least two more bits than the target."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal(1_000_000) * np.exp2(rng.integers(-120, 120, 1_000_000))
    f = x.astype(np.float32)
    exact = f.astype(np.float64) == x
    toward0 = np.where(np.abs(f.astype(np.float64)) > np.abs(x),
                       np.nextafter(f, np.float32(0)), f).astype(np.float32)
    bits = toward0.view(np.uint32) | np.where(exact, 0, 1).astype(np.uint32)
    bits = np.where(exact, f.view(np.uint32), bits)
    rne = ((bits.astype(np.uint64) + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(orc.encode(BF16, x), rne)


# --------------------------------------------------------------------------------------
# The experiment of "Tiling a matmul", section "Code": tiled vs naive on 32 x 32.
# --------------------------------------------------------------------------------------
def test_tiled_vs_naive_printed_loads(orc):
    """The page's experiment: 32 x 32 operands of U[0,1) doubles, the tiled loop against
    the naive one at tiles 1, 4 and 16.  The element loads it prints depend only on n and
    t (2 n^3 / t); the errors it prints are a few 1e-15.  The operands here come from this
    repository's seeded stream (the counts do not depend on the data)."""
    g = golden("tiling_a_matmul_code_output.json")["small_case"]
    n = g["n"]
    s = Stream(32)
    A = s.unit(n * n).reshape(n, n)
    B = s.unit(n * n).reshape(n, n)
    naive = orc.gemm_f64(A, B, B_KN)        # the page's product is A x B with B [K, N]
    assert np.allclose(naive, A @ B, rtol=0, atol=1e-13)
    for row in g["rows"]:
        C, loads = orc.tiled_f64(A, B, row["tile"])
        assert loads == row["loads"]
        err = np.max(np.abs(C - naive))
        # only the magnitude of the printed errors is fixed: their digits depend on the
        # data and on the summation of the page's reference product
        assert err <= 1e-14
    # With t = 1 every partial holds one product, so the tiled order is the naive order.
    C1, _ = orc.tiled_f64(A, B, 1)
    assert np.array_equal(C1, naive)


def test_tiled_vs_naive_dyadic_bitwise(orc):
    rng = np.random.default_rng(5)
    A = rng.integers(-64, 65, (32, 32)) / 64.0
    B = rng.integers(-64, 65, (32, 32)) / 64.0
    naive = orc.gemm_f64(A, B, B_KN)
    for t in (1, 2, 4, 8, 16, 32):
        C, loads = orc.tiled_f64(A, B, t)
        assert loads == 2 * 32 ** 3 // t
        assert np.array_equal(C, naive)     # every partial sum is exact


# --------------------------------------------------------------------------------------
# Closed forms and invariants of the 16-bit product.
# --------------------------------------------------------------------------------------
def _rand_bits(dtype, shape, seed, dist="uniform"):
    return Stream(seed).matrix(shape, dtype, dist)


def _one_bits(dtype):
    return np.uint16(0x3C00 if dtype == F16 else 0x3F80)


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("layout", [B_NK, B_KN])
def test_identity(orc, dtype, layout):
    K = 48
    eye = np.where(np.eye(K, dtype=bool), _one_bits(dtype), np.uint16(0)).astype(np.uint16)
    Bnk = _rand_bits(dtype, (37, K), 3)
    Bst = Bnk if layout == B_NK else np.ascontiguousarray(Bnk.T)
    C = orc.gemm(dtype, eye, Bst, layout)          # C = I x B^T = B^T
    assert np.array_equal(C, Bnk.T)
    A = _rand_bits(dtype, (29, K), 4)
    C2 = orc.gemm(dtype, A, eye, layout)           # C = A x I = A
    assert np.array_equal(C2, A)


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("K", [1, 7, 512, 1000])
def test_all_ones(orc, dtype, K):
    one = _one_bits(dtype)
    A = np.full((5, K), one, dtype=np.uint16)
    B = np.full((6, K), one, dtype=np.uint16)
    C = orc.gemm(dtype, A, B, B_NK)
    assert np.all(orc.decode(dtype, C) == float(K))


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_k_zero_and_empty(orc, dtype):
    A = np.zeros((3, 0), dtype=np.uint16)
    B = np.zeros((4, 0), dtype=np.uint16)
    C = orc.gemm(dtype, A, B, B_NK)
    assert C.shape == (3, 4) and np.all(C == 0)    # +0.0: the empty sum
    C0 = orc.gemm(dtype, np.zeros((0, 5), np.uint16), np.zeros((4, 5), np.uint16), B_NK)
    assert C0.shape == (0, 4)


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("layout", [B_NK, B_KN])
def test_tiny_shapes_brute_force_exact(orc, dtype, layout):
    """Every tiny product equals the correctly rounded exact rational sum."""
    frac_bits, emin, emax = (10, -14, 15) if dtype == F16 else (7, -126, 127)
    rng = np.random.default_rng(99 + dtype + 2 * layout)
    for _ in range(60):
        M, N, K = (int(v) for v in rng.integers(1, 7, 3))
        A = _rand_bits(dtype, (M, K), int(rng.integers(1 << 30)))
        Bnk = _rand_bits(dtype, (N, K), int(rng.integers(1 << 30)))
        Bst = Bnk if layout == B_NK else np.ascontiguousarray(Bnk.T)
        C = orc.gemm(dtype, A, Bst, layout)
        Ad = orc.decode(dtype, A)
        Bd = orc.decode(dtype, Bnk)
        for m in range(M):
            for n in range(N):
                s = sum(Fraction(float(Ad[m, k])) * Fraction(float(Bd[n, k]))
                        for k in range(K))
                want = _exact_round(s, frac_bits, emin, emax)
                got = Fraction(float(orc.decode(dtype, C[m:m + 1, n:n + 1])[0, 0]))
                assert got == want, (M, N, K, m, n)


def test_one_by_one_f16_is_ieee_multiply(orc):
    """A 1x1x1 fp16 product is the correctly rounded IEEE fp16 multiply."""
    rng = np.random.default_rng(3)
    a = rng.integers(0, 65536, 20000).astype(np.uint16)
    b = rng.integers(0, 65536, 20000).astype(np.uint16)
    fa, fb = a.view(np.float16), b.view(np.float16)
    ok = np.isfinite(fa) & np.isfinite(fb)
    a, b, fa, fb = a[ok], b[ok], fa[ok], fb[ok]
    with np.errstate(all="ignore"):
        want = (fa * fb)                          # numpy: correctly rounded fp16 multiply
    for i in range(0, a.size, 997):
        C = orc.gemm(F16, a[i:i + 1].reshape(1, 1), b[i:i + 1].reshape(1, 1), B_NK)
        g = C.view(np.float16)[0, 0]
        w = want[i]
        assert (np.isnan(g) and np.isnan(w)) or g == w, (hex(a[i]), hex(b[i]))


def test_f16_exact_integer_audit(orc):
    """For fp16 inputs in [-1, 1] every value is an integer multiple of 2^-24, so each sum
    is an exact integer multiple of 2^-48 (int64 holds it for K <= 2^14).  Rounded
    exactly to fp16, it must equal the oracle's fp64 sum rounded once."""
    w = WORKLOADS["f16_512"]
    A, B = w.generate()
    Ai = (A.view(np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)
    Bi = (B.view(np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)
    S = Ai @ Bi.T                                # exact integer matmul: |S| < 2^57
    C = orc.gemm(F16, A, B, B_NK)
    got = C.ravel().tolist()
    for i, s in enumerate(S.ravel().tolist()):
        mag = abs(s)
        step = max(mag.bit_length() - 11, 24)    # fp16 step at |S|, in units of 2^-48
        r, rem = divmod(mag, 1 << step)
        half = 1 << (step - 1)
        if rem > half or (rem == half and r & 1):
            r += 1
        exact = (-1.0 if s < 0 else 1.0) * r * 2.0 ** (step - 48)
        want = int(np.float16(exact).view(np.uint16))   # exact value, representable
        if s == 0:
            want = 0                               # +0.0 from +0.0 + exact zero products
        assert got[i] == want, (i, s)


def test_bf16_exact_python_ints(orc):
    """bf16 on a small case: exact sums with Python integers (arbitrary precision)."""
    M, N, K = 9, 7, 64
    A = _rand_bits(BF16, (M, K), 21)
    B = _rand_bits(BF16, (N, K), 22)
    C = orc.gemm(BF16, A, B, B_NK)
    Ad, Bd = orc.decode(BF16, A), orc.decode(BF16, B)
    for m in range(M):
        for n in range(N):
            s = sum(Fraction(float(Ad[m, k])) * Fraction(float(Bd[n, k])) for k in range(K))
            want = _exact_round(s, 7, -126, 127)
            got = Fraction(float(orc.decode(BF16, C[m:m + 1, n:n + 1])[0, 0]))
            assert got == want


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_metamorphic(orc, dtype):
    M, N, K = 33, 45, 70
    A = _rand_bits(dtype, (M, K), 31)
    B = _rand_bits(dtype, (N, K), 32)
    C = orc.gemm(dtype, A, B, B_NK)
    # swapping the operands gives the transpose, bit for bit (same products, same order)
    assert np.array_equal(orc.gemm(dtype, B, A, B_NK), C.T)
    # the two storage orders of the same logical B give the same bits
    assert np.array_equal(orc.gemm(dtype, A, np.ascontiguousarray(B.T), B_KN), C)
    # negating A negates C (sign bit flips; zeros may carry either sign)
    Cn = orc.gemm(dtype, A ^ np.uint16(0x8000), B, B_NK)
    assert np.array_equal(orc.decode(dtype, Cn), -orc.decode(dtype, C))
    # scaling A by 2 scales every fp64 sum by 2 exactly
    Ad = orc.decode(dtype, A) * 2.0
    A2 = orc.encode(dtype, Ad)
    _, S1 = orc.gemm(dtype, A, B, B_NK, want_sums=True)
    _, S2 = orc.gemm(dtype, A2, B, B_NK, want_sums=True)
    assert np.array_equal(S2, 2.0 * S1)


def test_threads_do_not_change_bits(orc):
    w = WORKLOADS["f16_512"]
    A, B = w.generate()
    c1 = orc.gemm(F16, A[:96], B[:80], B_NK, nthreads=1)
    c8 = orc.gemm(F16, A[:96], B[:80], B_NK, nthreads=8)
    assert np.array_equal(c1, c8)


@pytest.mark.parametrize("layout", [B_NK, B_KN])
def test_entries_and_rows_match_full(orc, layout):
    dtype = F16
    M, N, K = 70, 90, 130
    A = _rand_bits(dtype, (M, K), 41)
    Bnk = _rand_bits(dtype, (N, K), 42)
    Bst = Bnk if layout == B_NK else np.ascontiguousarray(Bnk.T)
    C, S = orc.gemm(dtype, A, Bst, layout, want_sums=True)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, M, 500)
    cols = rng.integers(0, N, 500)
    ce, se = orc.gemm_entries(dtype, A, Bst, layout, rows, cols)
    assert np.array_equal(ce, C[rows, cols])
    assert np.array_equal(se, S[rows, cols])
    assert np.array_equal(orc.gemm_rows(dtype, A, Bst, layout, 13, 29), C[13:29])


def test_numpy_matmul_agrees(orc):
    """The fp64 sums agree with numpy's matmul of the decoded inputs (a library routine
    that sums in another order) to fp64 rounding level."""
    w = WORKLOADS["f16_4000x3000x1000_kn"]
    A, B = w.generate()
    A, B = A[:64], B[:, :48]
    _, S = orc.gemm(F16, A, B, B_KN, want_sums=True)
    ref = orc.decode(F16, A) @ orc.decode(F16, B)
    assert np.allclose(S, ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------------
# The input generator (shared by both sides).
# --------------------------------------------------------------------------------------
def test_splitmix64_published_vector():
    # SplitMix64 from state 0: the first outputs of the reference generator.
    got = [int(v) for v in splitmix64(0, 0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_generator_rounding_and_ranges():
    s = Stream(1)
    x = s.uniform_pm1(100000)
    assert x.min() >= -1.0 and x.max() < 1.0
    bits = round_to_bf16_bits(x[x != 0])
    import torch
    via_torch = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    # round-to-nearest: within half a bf16 step of the draw
    err = np.abs(via_torch - x[x != 0])
    assert np.all(err <= np.abs(x[x != 0]) * 2.0 ** -8)
    z = Stream(4).normal(200000, 0.5)
    assert abs(z.std() - 0.5) < 0.01 and abs(z.mean()) < 0.01


def test_workloads_are_deterministic():
    w = WORKLOADS["f16_4000x3000x1000_kn"]
    a1, b1 = w.generate()
    a2, b2 = w.generate()
    assert a1.shape == (4000, 1000) and b1.shape == (1000, 3000)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)
