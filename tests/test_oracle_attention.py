"""Pins of the oracle's tiled Direct-P / FP8-P forward.

The pages print no worked example, so the attention oracle is pinned by
closed forms, a hand-derived probability-code case, invariants, and a
construction on which the quantized forward must equal textbook softmax
attention exactly (integer log2 scores whose 32-key blocks span at most four
consecutive integers: every 2**(t - m' - e) is then an exact E2M1 value).
"""

import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import quant as Q
from oracle import formats as F

LN2 = math.log(2.0)


def _integer_score_case(rng, nq, Nk, span, causal=False, growth=None):
    """q_raw, k_raw with integer scores S = q . k: S[i, j] =
    base[i, j % 64] + tile(j) * slope[i], with base values in
    {M_b, M_b-1, .., M_b-span+1} for each 32-key half of the 64-period and
    row.  D = 65."""
    D = 65
    q = np.zeros((nq, D))
    for i in range(nq):
        for half in range(2):
            M = rng.integers(-20, 21)
            q[i, 32 * half:32 * half + 32] = M - rng.integers(0, span, 32)
    q[:, 64] = growth if growth is not None else rng.integers(-3, 4, nq)
    k = np.zeros((Nk, D))
    k[np.arange(Nk), np.arange(Nk) % 64] = 1.0
    k[:, 64] = np.arange(Nk) // 128
    return q, k


@pytest.mark.parametrize("Nk", [32, 100, 128, 300, 517])
@pytest.mark.parametrize("causal", [False, True])
def test_directp_equals_exact_softmax_on_integer_scores(Nk, causal):
    rng = np.random.default_rng(Nk + causal)
    nq = Nk if causal else 37
    q, k = _integer_score_case(rng, nq, Nk, span=4)
    v = rng.standard_normal((Nk, 16))
    # sigma = ln 2 gives t = S in log2 units (c = sigma * log2 e * gq * gk = 1).
    O, lse = A.attn_lowp_head(q, k, 1.0, 1.0, v, LN2, "mxfp4", causal)
    Oe, lsee = A.attn_exact_head(q, k, v, LN2, causal)
    np.testing.assert_allclose(O, Oe, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lsee, rtol=1e-12, atol=1e-12)


def test_directp_integer_scores_detect_lossy_span():
    # a span of 5 integers inside a block makes 2**-4 * 4 = 0.25 round to 0:
    # the quantized forward must then differ from exact softmax.
    rng = np.random.default_rng(9)
    q, k = _integer_score_case(rng, 16, 256, span=8)
    v = rng.standard_normal((256, 8))
    O, _ = A.attn_lowp_head(q, k, 1.0, 1.0, v, LN2, "mxfp4")
    Oe, _ = A.attn_exact_head(q, k, v, LN2)
    assert np.abs(O - Oe).max() > 1e-6


@pytest.mark.parametrize("Nk", [64, 300])
def test_fp8p_equals_exact_softmax_on_integer_scores(Nk):
    # E4M3 holds 2**x exactly for integer x >= -9; keep every tile's scores
    # within 9 of its running max (slope >= 0 keeps old tiles at most 3+0 below).
    rng = np.random.default_rng(Nk)
    q, k = _integer_score_case(rng, 23, Nk, span=4, growth=0)
    for i in range(q.shape[0]):       # both halves share one max per row
        q[i, :64] = 5 - rng.integers(0, 6, 64)
    v = rng.standard_normal((Nk, 8))
    O, lse = A.attn_lowp_head(q, k, 1.0, 1.0, v, LN2, "fp8")
    Oe, lsee = A.attn_exact_head(q, k, v, LN2)
    np.testing.assert_allclose(O, Oe, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lsee, rtol=1e-12, atol=1e-12)


def test_hand_derived_probability_codes():
    # One query, one key per score: q_raw = 1, k_raw = t, sigma chosen so that
    # c = 1.  Block 0 holds the row max (x = 0 -> e = -2, values 2**(x+2)).
    # Block 1's max is x = -1.3 -> floor = -2 -> e = -4, values 2**(x+4).
    xs0 = [0.0, -0.5, -1.0, -1.5, -2.0, -2.5, -3.0, -3.9, -0.3, -0.2, -0.15, -4.5]
    # 2**(x+2): 4->6, 2.83->3(c5), 2->c4, 1.41->1.5(c3), 1->c2, .71->.5(c1),
    # .5->c1, .268->.5(c1), 3.25->3(c5), 3.48->3(c5), 3.61->4(c6), .177->0
    want0 = [6, 5, 4, 3, 2, 1, 1, 1, 5, 5, 6, 0]
    xs1 = [-1.3, -1.7, -2.7, -4.6, -6.0]
    # 2**(x+4): 6.50->6(c7, clipped), 4.92->4(c6), 2.46->2(c4), .66->.5(c1), .25->0 (tie)
    want1 = [7, 6, 4, 1, 0]
    t = np.full(64, -50.0)
    t[:len(xs0)] = xs0
    t[32:32 + len(xs1)] = xs1
    sigma = 1.0 / A.LOG2E
    O, lse, pc, pe = A.attn_lowp_head(np.ones((1, 1)), t[:, None], 1.0, 1.0,
                                      np.ones((64, 1)), sigma, "mxfp4", return_p=True)
    assert pe[0].tolist() == [125, 123]
    assert pc[0, :len(xs0)].tolist() == want0
    assert pc[0, 32:32 + len(xs1)].tolist() == want1
    # every -50 entry: 2**(-48) or 2**(-46) -> 0
    assert not pc[0, len(xs0):32].any() and not pc[0, 32 + len(xs1):].any()


def test_closed_form_zero_query():
    # Q = 0: all t = 0, every block has e = -2 and code 6 (4.0) -> p = 1,
    # l = Nk, O = mean of V, LSE = ln(Nk).
    rng = np.random.default_rng(11)
    Nk = 300
    v = rng.standard_normal((Nk, 4))
    for pf in ("mxfp4", "fp8"):
        O, lse = A.attn_lowp_head(np.zeros((3, 8)), rng.standard_normal((Nk, 8)),
                                  0.5, 0.25, v, 0.3, pf)
        np.testing.assert_allclose(O, np.broadcast_to(v.mean(0), O.shape), rtol=1e-13)
        np.testing.assert_allclose(lse, math.log(Nk), rtol=1e-15)


def test_closed_form_single_key_and_causal_first_row():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((5, 8))
    k = rng.standard_normal((5, 8))
    v = rng.standard_normal((5, 3))
    gq, gk, sigma = np.float32(0.75), np.float32(1.5), 0.2
    O, lse = A.attn_lowp_head(q, k[:1], gq, gk, v[:1], sigma, "mxfp4")
    np.testing.assert_allclose(O, np.broadcast_to(v[0], O.shape), rtol=1e-15)
    np.testing.assert_allclose(lse, sigma * float(gq) * float(gk) * (q @ k[0]), rtol=1e-12)
    O, lse = A.attn_lowp_head(q, k, gq, gk, v, sigma, "fp8", causal=True)
    np.testing.assert_allclose(O[0], v[0], rtol=1e-15)
    np.testing.assert_allclose(lse[0], sigma * float(gq) * float(gk) * (q[0] @ k[0]), rtol=1e-12)


def _quantized_head(rng, nq, Nk, D):
    x = rng.standard_normal((nq + Nk, D)).astype(np.float32)
    qc, qs, gq = Q.quant_nvfp4(x[:nq])
    kc, ks, gk = Q.quant_nvfp4(x[nq:])
    return Q.dequant_nvfp4_raw(qc, qs), gq, Q.dequant_nvfp4_raw(kc, ks), gk, x


def test_invariant_v_scaling_is_exact():
    rng = np.random.default_rng(13)
    qr, gq, kr, gk, _ = _quantized_head(rng, 20, 333, 64)
    v = rng.standard_normal((333, 64))
    O1, l1 = A.attn_lowp_head(qr, kr, gq, gk, v, 0.125, "mxfp4")
    O2, l2 = A.attn_lowp_head(qr, kr, gq, gk, 2 * v, 0.125, "mxfp4")
    np.testing.assert_array_equal(O2, 2 * O1)
    np.testing.assert_array_equal(l1, l2)


def test_invariant_query_scaling_through_quantization():
    # Q <- 2Q keeps codes and block scales and doubles g; with sigma <- sigma/2
    # every t is bitwise the same, hence the same codes and O.
    rng = np.random.default_rng(14)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    kx = rng.standard_normal((200, 64)).astype(np.float32)
    v = rng.standard_normal((200, 64))
    kc, ks, gk = Q.quant_nvfp4(kx)
    outs = []
    for f, sig in ((1, 0.125), (2, 0.0625)):
        qc, qs, gq = Q.quant_nvfp4(x * np.float32(f))
        outs.append(A.attn_lowp_head(Q.dequant_nvfp4_raw(qc, qs), Q.dequant_nvfp4_raw(kc, ks),
                                     gq, gk, v, sig, "mxfp4", return_p=True))
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)


def test_denominator_is_sum_of_rounded_probabilities():
    # single tile: l = sum of dequantized P, so LSE = ln2 * (m + log2 sum p_hat)
    rng = np.random.default_rng(15)
    qr, gq, kr, gk, _ = _quantized_head(rng, 8, 128, 64)
    v = np.eye(128)                                   # O = p_hat / l
    O, lse, pc, pe = A.attn_lowp_head(qr, kr, gq, gk, v, 0.125, "mxfp4", return_p=True)
    p_hat = F.e2m1_decode(pc) * np.repeat(F.e8m0_decode(pe), 32, axis=1)
    l = p_hat.sum(1)
    np.testing.assert_allclose(O, p_hat / l[:, None], rtol=1e-14)
    t = 0.125 * A.LOG2E * float(gq) * float(gk) * (qr @ kr.T)
    np.testing.assert_allclose(lse, LN2 * (t.max(1) + np.log2(l)), rtol=1e-13)


def test_quantization_error_is_small_against_unquantized_attention():
    # Not parity: a sanity bound on the total quantization error (a dropped
    # term, sign or transposition would give O(1) errors).
    rng = np.random.default_rng(16)
    qr, gq, kr, gk, x = _quantized_head(rng, 64, 512, 64)
    v = rng.standard_normal((512, 64)).astype(np.float32)
    vc, ve = Q.quant_v_mxfp4(v[:, None, :])
    vh = Q.dequant_v_mxfp4(vc, ve)[:, 0, :]
    O, lse = A.attn_lowp_head(qr, kr, gq, gk, vh, 0.125, "mxfp4")
    Oe, lsee = A.attn_exact_head(x[:64], x[64:], v, 0.125)
    rel = np.linalg.norm(O - Oe) / np.linalg.norm(Oe)
    assert rel < 0.25, rel
    assert np.abs(lse - lsee).max() < 0.1


def test_empty_keys():
    O, lse = A.attn_lowp_head(np.ones((2, 4)), np.zeros((0, 4)), 1, 1, np.zeros((0, 3)), 1.0)
    assert O.shape == (2, 3) and not O.any() and np.all(np.isneginf(lse))


def test_hand_derived_tile_boundary_at_128_keys():
    # t: key 0 = 0.0, key 64 = 0.3, key 128 = 1.0, all others -1000: a block
    # holding only those gets e = -127 and 2**(-1000 + 127) -> code 0.
    # Tile 0 (keys 0..127) has m' = 0.3: block 0's xmax = -0.3 -> e = -3 and
    # key 0 -> 2**(0 - 0.3 + 3) = 6.50 -> code 7 (6.0, clipped), p = 0.75;
    # block 2's xmax = 0 -> e = -2, key 64 -> 4.0 (code 6), p = 1.
    # Tile 1 has m' = 1.0, alpha = 2**(0.3 - 1.0); key 128 -> code 6, e = -2, p = 1.
    # (A 64-key tile would give key 0 code 6; a 256-key tile would give e = -3
    # with code 6.)  With V = identity, O[j] = p_j * 2**(m_j - m) / l.
    Nk = 160
    t = np.full(Nk, -1000.0)
    t[[0, 64, 128]] = [0.0, 0.3, 1.0]
    sigma = 1.0 / A.LOG2E
    O, lse, pc, pe = A.attn_lowp_head(np.ones((1, 1)), t[:, None], 1.0, 1.0,
                                      np.eye(Nk), sigma, "mxfp4", return_p=True)
    assert pc[0, [0, 64, 128]].tolist() == [7, 6, 6]
    assert pe[0].tolist() == [124, 0, 125, 0, 125]
    assert np.flatnonzero(pc[0]).tolist() == [0, 64, 128]
    a = 2.0 ** (0.3 - 1.0)
    l = (0.75 + 1.0) * a + 1.0
    np.testing.assert_allclose(O[0, [0, 64, 128]], [0.75 * a / l, a / l, 1.0 / l], rtol=1e-14)
    np.testing.assert_allclose(lse[0], LN2 * (1.0 + math.log2(l)), rtol=1e-14)
