"""Pins of the oracle's exp-free log-linear probability casts (oracle.loglin)
and of the forward that uses them (attn_lowp_head(..., encoder="loglin")).

The related pages give only abstracts, so the cast is pinned by what its
definition fixes independently of the code that computes it: Mitchell's
piecewise-linear 2**y (evaluated from floor and fraction, not from the code
integer), agreement with the already pinned RNE E2M1 encoder where the two
coincide, hand-derived codes, and integer-score attention cases on which the
cast is exact, so that the forward must equal textbook softmax attention.
"""

import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import formats as F
from oracle.loglin import loglin_encode

LN2 = math.log(2.0)


def _mitchell(y, mbits):
    """2**n * (1 + r / 2**M), n = floor(y), r = 2**M (y - n) rounded half to even."""
    n = np.floor(y)
    r = np.rint(np.ldexp(y - n, mbits))
    return np.ldexp(1.0 + np.ldexp(r, -mbits), n.astype(np.int64))


def _decode(codes, fmt):
    return F.e4m3_decode(codes) if fmt == "e4m3" else F.e2m1_decode(codes)


def test_e4m3_integer_log_points_are_exact():
    for k in range(-6, 1):
        assert _decode(loglin_encode(float(k), "e4m3"), "e4m3") == 2.0 ** k
    # below the smallest normal the cast leaves 0 at integer points
    assert loglin_encode(np.array([-7.0, -8.0, -30.0, -np.inf]), "e4m3").tolist() == [0, 0, 0, 0]


def test_e2m1_integer_log_points_are_exact():
    for k in range(0, 3):
        assert _decode(loglin_encode(float(k), "e2m1"), "e2m1") == 2.0 ** k
    assert loglin_encode(np.array([-1.0, -2.0, -np.inf]), "e2m1").tolist() == [0, 0, 0]


def test_e4m3_normal_range_is_mitchell():
    # every multiple of 1/64 in [-6, 0] (ties at odd multiples of 1/16)
    y = np.arange(-6 * 64, 1) / 64.0
    got = _decode(loglin_encode(y, "e4m3"), "e4m3")
    np.testing.assert_array_equal(got, _mitchell(y, 3))


def test_e2m1_normal_range_is_mitchell_and_rne_of_it():
    # y in [0, 2.75): below the saturation of code 7
    y = np.arange(0, 11 * 16) / 64.0
    got = _decode(loglin_encode(y, "e2m1"), "e2m1")
    np.testing.assert_array_equal(got, _mitchell(y, 1))
    # on n >= 0 the cast equals the RNE E2M1 encoding of 2**n * (1 + f)
    # (one mantissa bit per binade), saturation included up to y < 3
    y = np.arange(0, 3 * 64) / 64.0
    n = np.floor(y)
    lin = np.ldexp(1.0 + (y - n), n.astype(np.int64))
    want = F.e2m1_decode(F.e2m1_encode(lin))
    np.testing.assert_array_equal(_decode(loglin_encode(y, "e2m1"), "e2m1"), want)


def test_hand_derived_codes():
    # E4M3: 8 (y + 7): y = -0.5 -> 52 (0x34 = 1.5 * 2**-1 = 0.75)
    #       y = -1/16 -> 55.5 -> 56 (tie, even); y = -3/16 -> 54.5 -> 54
    #       y = -6.9 -> 0.8 -> 1 (subnormal 2**-9); y = -6.95 -> 0.4 -> 0
    ys = [-0.5, -1 / 16, -3 / 16, -6.9, -6.95, 0.0]
    assert loglin_encode(np.array(ys), "e4m3").tolist() == [52, 56, 54, 1, 0, 56]
    assert F.e4m3_decode(52) == 0.75
    # E2M1: 2 (y + 1): y = 2.9 -> 7.8 -> 8 -> clamp 7 (6.0); y = 2.25 -> 6.5 -> 6
    #       y = -0.3 -> 1.4 -> 1 (0.5); y = -0.25 -> 1.5 -> 2 (tie, even)
    #       y = -0.75 -> 0.5 -> 0 (tie, even); y = 0.6 -> 3.2 -> 3 (1.5)
    ys = [2.9, 2.25, -0.3, -0.25, -0.75, 0.6]
    assert loglin_encode(np.array(ys), "e2m1").tolist() == [7, 6, 1, 2, 0, 3]


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_monotone_and_bounded(fmt):
    y = np.linspace(-20, 4, 100001)
    c = loglin_encode(y, fmt).astype(np.int64)
    assert np.all(np.diff(c) >= 0)
    assert c.max() == (0x7E if fmt == "e4m3" else 7) or fmt == "e4m3"
    assert c.min() == 0


def _integer_score_case(rng, nq, Nk, span, growth):
    """Integer scores S = q . k (D = 65): each 32-key block of a row takes
    values from {M, .., M - span + 1}; key tile j adds j * growth[i]."""
    D = 65
    q = np.zeros((nq, D))
    for i in range(nq):
        for half in range(2):
            M = rng.integers(-20, 21)
            q[i, 32 * half:32 * half + 32] = M - rng.integers(0, span, 32)
    q[:, 64] = growth
    k = np.zeros((Nk, D))
    k[np.arange(Nk), np.arange(Nk) % 64] = 1.0
    k[:, 64] = np.arange(Nk) // 128
    return q, k


@pytest.mark.parametrize("Nk", [32, 200, 517])
@pytest.mark.parametrize("causal", [False, True])
def test_efq_equals_exact_softmax_on_integer_scores(Nk, causal):
    # y = t - (block max) + 2 takes the values 2, 1, 0 only: codes 6, 4, 2
    # hold 4, 2, 1 exactly, so the forward is textbook softmax attention.
    rng = np.random.default_rng(100 + Nk + causal)
    nq = Nk if causal else 19
    q, k = _integer_score_case(rng, nq, Nk, span=3, growth=rng.integers(-3, 4, nq))
    v = rng.standard_normal((Nk, 8))
    O, lse = A.attn_lowp_head(q, k, 1.0, 1.0, v, LN2, "mxfp4", causal, encoder="loglin")
    Oe, lsee = A.attn_exact_head(q, k, v, LN2, causal)
    np.testing.assert_allclose(O, Oe, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lsee, rtol=1e-12, atol=1e-12)


def test_efq_drops_what_direct_p_keeps():
    # span 4 puts y = -1 in blocks: RNE keeps 0.5 there (Direct-P stays exact),
    # the cast gives code 0 (2 * (y + 1) = 0)
    rng = np.random.default_rng(7)
    q, k = _integer_score_case(rng, 16, 256, span=4, growth=0)
    v = rng.standard_normal((256, 8))
    Oe, _ = A.attn_exact_head(q, k, v, LN2)
    Od, _ = A.attn_lowp_head(q, k, 1.0, 1.0, v, LN2, "mxfp4")
    Ol, _ = A.attn_lowp_head(q, k, 1.0, 1.0, v, LN2, "mxfp4", encoder="loglin")
    np.testing.assert_allclose(Od, Oe, rtol=1e-12, atol=1e-12)
    assert np.abs(Ol - Oe).max() > 1e-3


@pytest.mark.parametrize("Nk", [64, 300])
def test_fp8_cast_equals_exact_softmax_on_integer_scores(Nk):
    # every live x = t - m' in [-5, 0] and integer: E4M3 code 8 (x + 7) holds
    # 2**x exactly.  Both halves share one max per row, no growth.
    rng = np.random.default_rng(200 + Nk)
    q, k = _integer_score_case(rng, 23, Nk, span=4, growth=0)
    for i in range(q.shape[0]):
        q[i, :64] = 5 - rng.integers(0, 6, 64)
    v = rng.standard_normal((Nk, 8))
    O, lse = A.attn_lowp_head(q, k, 1.0, 1.0, v, LN2, "fp8", encoder="loglin")
    Oe, lsee = A.attn_exact_head(q, k, v, LN2)
    np.testing.assert_allclose(O, Oe, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lsee, rtol=1e-12, atol=1e-12)


def test_fp8_cast_is_mitchell_weighted_softmax():
    # One tile, scores on the 1/8 grid: P = Mitchell 2**x, O = P v / sum P,
    # LSE = ln2 (m + log2 sum P), written out from the closed form.
    rng = np.random.default_rng(31)
    Nk = 128
    t = -rng.integers(0, 48, Nk) / 8.0
    t[5] = 0.0
    v = rng.standard_normal((Nk, 6))
    O, lse, pc, _ = A.attn_lowp_head(np.ones((1, 1)), t[:, None], 1.0, 1.0, v, 1.0 / A.LOG2E, "fp8",
                                     encoder="loglin", return_p=True)
    p = _mitchell(t, 3)
    np.testing.assert_array_equal(F.e4m3_decode(pc[0]), p)
    np.testing.assert_allclose(O[0], p @ v / p.sum(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0], LN2 * math.log2(p.sum()), rtol=1e-13)


def test_efq_block_exponent_is_direct_p_rule():
    # the E8M0 bytes of the cast are those of Direct-P; only codes differ
    rng = np.random.default_rng(41)
    q = rng.standard_normal((9, 16))
    k = rng.standard_normal((300, 16))
    v = rng.standard_normal((300, 4))
    _, _, pc0, pe0 = A.attn_lowp_head(q, k, 1.0, 1.0, v, 0.7, "mxfp4", return_p=True)
    _, _, pc1, pe1 = A.attn_lowp_head(q, k, 1.0, 1.0, v, 0.7, "mxfp4", return_p=True, encoder="loglin")
    np.testing.assert_array_equal(pe0, pe1)
    assert (pc0 != pc1).mean() > 0.05
