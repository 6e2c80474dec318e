"""Pins of the acceptance rule every GPU parity claim rests on (-m "not gpu").

The rule: an element passes when it is finite and |gpu - oracle| <= 1e-3 * sqrt(K) + one
step ("ulp") of the output format at |oracle|.  The step is fixed by the formats
themselves -- IEEE binary16 (11 significant bits, smallest normal exponent -14) and
bfloat16 (8 significant bits, smallest normal exponent -126) -- so the pins below are
values of those formats, numpy's own spacing routine over every finite value, and
hand-worked cases of the bound, not a second copy of the formula.
"""
import numpy as np
import pytest

from tiled_dense_gemm_major_amd.inputs import BF16, F16, round_to_bf16_bits


# --------------------------------------------------------------------------------------
# ulp_out: the spacing of the output format.
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,x,want", [
    # zero: the subnormal spacing, 2^(emin - p + 1)
    (F16, 0.0, 2.0 ** -24), (BF16, 0.0, 2.0 ** -133),
    # one: 2^-(p-1)
    (F16, 1.0, 2.0 ** -10), (BF16, 1.0, 2.0 ** -7),
    # 30 lies in [16, 32): 2^(4 - p + 1)
    (F16, 30.0, 2.0 ** -6), (BF16, 30.0, 0.125),
    # the smallest normal number of each format
    (F16, 2.0 ** -14, 2.0 ** -24), (BF16, 2.0 ** -126, 2.0 ** -133),
    # subnormals share the smallest normal binade's spacing
    (F16, 2.0 ** -20, 2.0 ** -24), (F16, 2.0 ** -24, 2.0 ** -24),
    (BF16, 2.0 ** -130, 2.0 ** -133),
    # the largest finite numbers: 65504 = (2 - 2^-10) 2^15, (2 - 2^-7) 2^127
    (F16, 65504.0, 32.0), (BF16, (2.0 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** 120),
    # the sign does not matter; just below a power of two is the lower binade
    (F16, -1.0, 2.0 ** -10), (F16, 1.0 - 2.0 ** -11, 2.0 ** -11),
])
def test_ulp_out_values(orc, dtype, x, want):
    assert orc.ulp_out(dtype, [x])[0] == want


def test_ulp_out_f16_every_finite_value_matches_numpy_spacing(orc):
    """For every finite fp16 value below the largest, the step up to the next value is
    numpy's float16 spacing."""
    bits = np.arange(0, 0x7C00, dtype=np.uint16)[:-1]      # 0 .. the largest finite - 1
    x = bits.view(np.float16)
    want = np.spacing(x).astype(np.float64)
    assert np.array_equal(orc.ulp_out(F16, x.astype(np.float64)), want)
    assert np.array_equal(orc.ulp_out(F16, -x.astype(np.float64)), want)


def test_ulp_out_bf16_every_finite_value_matches_scaled_f32_spacing(orc):
    """bfloat16 is float32 with 16 fraction bits dropped, so at every bfloat16 value its
    step is float32's spacing times 2^16 (numpy's float32 spacing routine)."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)[:-1]
    x = (bits << 16).view(np.float32)
    want = np.spacing(x).astype(np.float64) * 65536.0
    assert np.array_equal(orc.ulp_out(BF16, x.astype(np.float64)), want)


def test_ulp_out_non_finite_is_nan(orc):
    got = orc.ulp_out(F16, [np.inf, -np.inf, np.nan])
    assert np.all(np.isnan(got))


# --------------------------------------------------------------------------------------
# tolerance: 1e-3 * sqrt(K) + ulp(|oracle|), worked by hand.
# --------------------------------------------------------------------------------------
def test_tolerance_worked_values(orc):
    # K = 512: sqrt(512) = 22.627416997969522 -> 0.022627416997969522; at |oracle| = 1
    # the fp16 step is 2^-10 = 0.0009765625
    assert orc.tolerance(F16, 512, [1.0])[0] == pytest.approx(0.023603979497969522,
                                                             rel=1e-15)
    # K = 8192: sqrt(8192) = 90.50966799187808 -> 0.09050966799187808; at |oracle| = 30
    # the bf16 step is 0.125
    assert orc.tolerance(BF16, 8192, [30.0])[0] == pytest.approx(0.21550966799187808,
                                                                 rel=1e-15)
    # at an oracle of zero only the subnormal step is added
    assert orc.tolerance(BF16, 8192, [0.0])[0] == pytest.approx(
        0.09050966799187808 + 2.0 ** -133, rel=1e-15)
    # K = 10^6: 1e-3 * 1000 rounds to exactly 1.0
    assert orc.tolerance(BF16, 10 ** 6, [8.0])[0] == 1.0 + 2.0 ** -4
    # K = 0 (the empty sum): the bound is one step
    assert orc.tolerance(F16, 0, [1.0])[0] == 2.0 ** -10


# --------------------------------------------------------------------------------------
# compare: the element-wise decision.
# --------------------------------------------------------------------------------------
def _bits(dtype, values):
    values = np.asarray(values, dtype=np.float64)
    if dtype == F16:
        return values.astype(np.float16).view(np.uint16)
    return round_to_bf16_bits(values)


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_compare_bound_is_inclusive_at_k_zero(orc, dtype):
    step = 2.0 ** -10 if dtype == F16 else 2.0 ** -7
    want = _bits(dtype, [1.0, 1.0, 1.0])
    at = orc.compare(dtype, 0, _bits(dtype, [1.0, 1.0 + step, 1.0 - step / 2]), want)
    assert at["n_fail"] == 0 and at["max_err_over_tol"] == 1.0
    over = orc.compare(dtype, 0, _bits(dtype, [1.0, 1.0 + 2 * step, 1.0]), want)
    assert over["n_fail"] == 1 and over["first_fail"] == 1


def test_compare_bound_with_a_k_term(orc):
    # K = 10^6, oracle 8: bound 1 + 2^-4 = 1.0625.  9.0625 sits exactly on it; the next
    # bf16 value up, 9.125, is one step over
    want = _bits(BF16, [8.0, 8.0, 8.0, 8.0])
    got = _bits(BF16, [9.0, 9.0625, 6.9375, 9.125])
    res = orc.compare(BF16, 10 ** 6, got, want)
    assert res["n_fail"] == 1 and res["first_fail"] == 3
    assert res["max_err"] == 1.125


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_compare_fails_non_finite_results(orc, dtype):
    nan_bits = 0x7E00 if dtype == F16 else 0x7FC0
    inf_bits = 0x7C00 if dtype == F16 else 0x7F80
    want = _bits(dtype, [0.5, 0.5, 0.5, 0.5])
    got = want.copy()
    got[1] = nan_bits
    got[2] = inf_bits
    got[3] = inf_bits | 0x8000
    res = orc.compare(dtype, 4096, got, want)
    assert res["n_fail"] == 3 and res["first_fail"] == 1
    # an exact match of a finite value passes, whatever K
    assert orc.compare(dtype, 1, want, want)["n_fail"] == 0


def test_compare_fails_against_a_non_finite_oracle(orc):
    want = np.array([0x7C00, 0x7E00], dtype=np.uint16)         # +inf, NaN
    assert orc.compare(F16, 16, want, want)["n_fail"] == 2


# --------------------------------------------------------------------------------------
# attention_tolerance and compare_attention, worked by hand.
# --------------------------------------------------------------------------------------
def test_attention_tolerance_worked_case(orc):
    # one (batch, head), 3 keys, dim 2: column 0 holds 0.5, 0.5, -2 (max |v| = 2),
    # column 1 holds 0.25 everywhere (max |v| = 0.25)
    V = np.zeros((1, 3, 1, 2), dtype=np.uint16)
    V[0, :, 0, 0] = _bits(F16, [0.5, 0.5, -2.0])
    V[0, :, 0, 1] = _bits(F16, [0.25, 0.25, 0.25])
    orc_vals = np.ones((1, 3, 1, 2))
    tol = orc.attention_tolerance(V, True, orc_vals)
    # 4 * 2^-11 * 2 + 2^-10 = 2^-8 + 2^-10; 4 * 2^-11 * 0.25 + 2^-10 = 2^-11 + 2^-10
    assert np.all(tol[..., 0] == 2.0 ** -8 + 2.0 ** -10)
    assert np.all(tol[..., 1] == 2.0 ** -11 + 2.0 ** -10)


def test_compare_attention_decisions(orc):
    V = np.zeros((1, 2, 1, 1), dtype=np.uint16)
    V[0, :, 0, 0] = _bits(F16, [1.0, -1.0])         # tolerance 2^-9 + 2^-10 at |O| = 1
    want = _bits(F16, [1.0, 1.0]).reshape(1, 2, 1, 1)
    inside = _bits(F16, [1.0 + 2.0 ** -10 * 3, 1.0]).reshape(1, 2, 1, 1)
    assert orc.compare_attention(V, False, inside, want)["n_fail"] == 0
    outside = _bits(F16, [1.0 + 2.0 ** -10 * 4, 1.0]).reshape(1, 2, 1, 1)
    assert orc.compare_attention(V, False, outside, want)["n_fail"] == 1
    nan = want.copy()
    nan[0, 1, 0, 0] = 0x7E00
    res = orc.compare_attention(V, False, nan, want)
    assert res["n_fail"] == 1 and res["first_fail"] == 1

