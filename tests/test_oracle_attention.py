"""Pins for the attention oracle against what the page and the mathematics fix,
independent of the oracle's own code: closed forms (equal values, a single key, equal
scores, a known score gap), exact rational means, an independent log-sum-exp evaluation
in Python, and invariants (scaling V, swapping heads, the causal last row, permuted keys,
a common shift of every score)."""
import math
from fractions import Fraction

import numpy as np
import pytest

from tests.test_oracle_pins import _exact_round
from tiled_dense_gemm_major_amd.inputs import F16, Stream


def _qkv(shape, seed, sigma=1.0):
    s = Stream(seed)
    return tuple(s.matrix(shape, F16, "normal", sigma) for _ in range(3))


def _f16(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def _val(orc, bits):
    return orc.decode(F16, bits)


def _round_f16_exact(fr):
    r = _exact_round(fr, 10, -14, 15)
    return np.float16(float(r)).view(np.uint16)       # r is an fp16 value: exact


@pytest.mark.parametrize("causal", [False, True])
def test_equal_values_give_that_value(orc, causal):
    """Every key carries the same V row: any weighted average is that row."""
    B, S, H, D = 2, 37, 3, 16
    Q, K, _ = _qkv((B, S, H, D), 1)
    row = Stream(2).matrix((1, 1, H, D), F16, "normal", 1.0)
    V = np.broadcast_to(row, (B, S, H, D)).copy()
    O = orc.attention(Q, K, V, causal)
    assert np.array_equal(O, np.broadcast_to(row, (B, S, H, D)))


def test_first_causal_row_is_first_value(orc):
    """Under the causal mask the first query sees only the first key: weight exactly 1."""
    Q, K, V = _qkv((2, 9, 4, 32), 3)
    O = orc.attention(Q, K, V, True)
    assert np.array_equal(O[:, 0], V[:, 0])


@pytest.mark.parametrize("causal", [False, True])
def test_equal_scores_give_exact_means(orc, causal):
    """K = 0 makes every score 0: the output is the plain mean of the allowed V rows
    (prefix means under the causal mask), checked against exact rational means rounded
    to fp16 by exact rational rounding."""
    B, S, H, D = 1, 12, 2, 8
    Q, _, V = _qkv((B, S, H, D), 4)
    K = np.zeros_like(Q)
    O = orc.attention(Q, K, V, causal)
    Vd = _val(orc, V)
    for h in range(H):
        for i in range(S):
            n = i + 1 if causal else S
            for d in range(D):
                mean = sum(Fraction(float(Vd[0, j, h, d])) for j in range(n)) / n
                assert O[0, i, h, d] == _round_f16_exact(mean), (h, i, d)


def test_known_score_gap_fixes_scale_and_base(orc):
    """Two keys whose scores differ by exactly 1 after the 1/sqrt(D) scale (q.k = 8 with
    D = 64): the weights are 1/(1+e) and e/(1+e).  A wrong scale (1/D, none) or base
    (2 instead of e) moves the output far outside the fp16 rounding."""
    D = 64
    Q = np.zeros((1, 2, 1, D), dtype=np.uint16)
    K = np.zeros_like(Q)
    V = np.zeros_like(Q)
    Q[0, :, 0, 0] = _f16(1.0)
    K[0, 1, 0, 0] = _f16(8.0)                        # s_1 - s_0 = 8 / sqrt(64) = 1
    V[0, 0, 0, :] = _f16(np.linspace(-2, 2, D))
    V[0, 1, 0, :] = _f16(np.linspace(3, -1, D))
    O, O64 = orc.attention(Q, K, V, False, want_f64=True)
    v0, v1 = _val(orc, V[0, 0, 0]), _val(orc, V[0, 1, 0])
    want = (v0 + math.e * v1) / (1.0 + math.e)
    assert np.allclose(O64[0, 0, 0], want, rtol=1e-14, atol=1e-14)
    assert np.allclose(O64[0, 1, 0], want, rtol=1e-14, atol=1e-14)


def _lse_reference(Qd, Kd, Vd, causal):
    """O by the log-sum-exp form, in plain Python floats with compensated sums:
    w_j = exp(s_j - lse), lse = log(sum_j exp(s_j)) (shifted by the max for range)."""
    B, S, H, D = Qd.shape
    out = np.empty_like(Qd)
    for b in range(B):
        for h in range(H):
            for i in range(S):
                n = i + 1 if causal else S
                s = [math.fsum(Qd[b, i, h, d] * Kd[b, j, h, d] for d in range(D)) / math.sqrt(D)
                     for j in range(n)]
                m = max(s)
                lse = m + math.log(math.fsum(math.exp(x - m) for x in s))
                w = [math.exp(x - lse) for x in s]
                for d in range(D):
                    out[b, i, h, d] = math.fsum(w[j] * Vd[b, j, h, d] for j in range(n))
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_log_sum_exp(orc, causal):
    B, S, H, D = 2, 7, 2, 8
    Q, K, V = _qkv((B, S, H, D), 5, sigma=1.5)
    _, O64 = orc.attention(Q, K, V, causal, want_f64=True)
    ref = _lse_reference(_val(orc, Q), _val(orc, K), _val(orc, V), causal)
    assert np.allclose(O64, ref, rtol=1e-12, atol=1e-13)


def test_matches_library_softmax(orc):
    """scipy's softmax and numpy's matrix products on a mid-size case."""
    special = pytest.importorskip("scipy.special")
    B, S, H, D = 1, 40, 3, 32
    Q, K, V = _qkv((B, S, H, D), 6)
    _, O64 = orc.attention(Q, K, V, True, want_f64=True)
    Qd, Kd, Vd = (_val(orc, x) for x in (Q, K, V))
    for h in range(H):
        sc = Qd[0, :, h, :] @ Kd[0, :, h, :].T / math.sqrt(D)
        sc[np.triu_indices(S, 1)] = -np.inf
        ref = special.softmax(sc, axis=1) @ Vd[0, :, h, :]
        assert np.allclose(O64[0, :, h, :], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(orc, causal):
    B, S, H, D = 2, 33, 3, 16
    Q, K, V = _qkv((B, S, H, D), 7)
    O, O64 = orc.attention(Q, K, V, causal, want_f64=True)
    # doubling V doubles the unrounded O exactly (every fp64 product and sum scales by 2),
    # and the rounded O wherever it is a normal fp16 number (below that the rounding
    # step does not double)
    V2 = _f16(_val(orc, V) * 2.0)
    O2, O2_64 = orc.attention(Q, K, V2, causal, want_f64=True)
    assert np.array_equal(O2_64, 2.0 * O64)
    normal = np.abs(O64) >= 2.0 ** -13
    assert np.array_equal(_val(orc, O2)[normal], 2.0 * _val(orc, O)[normal])
    # heads are independent: swapping two heads swaps their outputs
    perm = [2, 0, 1]
    Op = orc.attention(Q[:, :, perm], K[:, :, perm], V[:, :, perm], causal)
    assert np.array_equal(Op, O[:, :, perm])
    # the last query sees every key under either mask
    Of = orc.attention(Q, K, V, not causal)
    assert np.array_equal(Of[:, -1], O[:, -1])


def test_permuted_keys_and_shifted_scores(orc):
    """Without the mask the keys are a set: permuting them (with their values) leaves O;
    adding one constant to every score of a row (a dimension where every key holds 1 and
    the query some c) leaves the softmax -- both up to fp64 rounding."""
    B, S, H, D = 1, 24, 2, 16
    Q, K, V = _qkv((B, S, H, D), 8)
    _, O64 = orc.attention(Q, K, V, False, want_f64=True)
    perm = np.random.default_rng(0).permutation(S)
    _, Op = orc.attention(Q, K[:, perm], V[:, perm], False, want_f64=True)
    assert np.allclose(Op, O64, rtol=1e-13, atol=1e-14)
    K1, Q1, Q2 = K.copy(), Q.copy(), Q.copy()
    K1[..., 0] = _f16(1.0)
    Q1[..., 0] = _f16(0.0)
    Q2[..., 0] = _f16(3.0)
    _, Oa = orc.attention(Q1, K1, V, False, want_f64=True)
    _, Ob = orc.attention(Q2, K1, V, False, want_f64=True)
    assert np.allclose(Oa, Ob, rtol=1e-12, atol=1e-13)


def test_empty_and_argument_checks(orc):
    z = np.zeros((1, 0, 2, 8), dtype=np.uint16)
    assert orc.attention(z, z, z, True).shape == z.shape
    Q, K, V = _qkv((1, 5, 1, 8), 9)
    with pytest.raises(ValueError):
        orc.attention(Q, K[:, :4], V, True)
