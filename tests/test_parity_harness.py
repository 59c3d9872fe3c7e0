"""CPU tests of the parity machinery: the oracle's code-substitution and
pre-rounding hooks, and the near-tie check that decides whether a
probability code the kernel rounded differently from the oracle is valid."""

import math

import numpy as np
import pytest

from helpers import check_code_choices
from oracle import attention as A
from oracle import formats as F
from oracle.loglin import loglin_round

LN2 = math.log(2.0)


def _head(rng, nq=7, nk=300, d=16):
    return rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, 5))


@pytest.mark.parametrize("pf,enc", [("mxfp4", "exact"), ("mxfp4", "loglin"), ("fp8", "exact"), ("fp8", "loglin")])
def test_given_own_codes_is_identity(pf, enc):
    rng = np.random.default_rng(1)
    q, k, v = _head(rng)
    O, lse, pc, pe = A.attn_lowp_head(q, k, 1.0, 1.0, v, 0.6, pf, return_p=True, encoder=enc)
    O2, lse2 = A.attn_lowp_head(q, k, 1.0, 1.0, v, 0.6, pf, encoder=enc, p_given=(pc, pe))
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(lse, lse2)


def test_given_codes_closed_form_single_tile():
    # one tile, FP8 P: O = sum p v / sum p over the given codes' values,
    # LSE = ln2 (m + log2 sum p)
    rng = np.random.default_rng(2)
    t = -rng.uniform(0, 6, 100)
    t[3] = 0.0
    v = rng.standard_normal((100, 4))
    codes = rng.integers(0, 57, (1, 100)).astype(np.uint8)
    O, lse = A.attn_lowp_head(np.ones((1, 1)), t[:, None], 1.0, 1.0, v, 1.0 / A.LOG2E, "fp8", p_given=(codes, None))
    p = F.e4m3_decode(codes[0])
    np.testing.assert_allclose(O[0], p @ v / p.sum(), rtol=1e-13)
    np.testing.assert_allclose(lse[0], LN2 * math.log2(p.sum()), rtol=1e-12)


def test_pre_values_are_what_is_rounded():
    rng = np.random.default_rng(3)
    q, k, v = _head(rng, nq=9, nk=290)
    for pf in ("mxfp4", "fp8"):
        for enc in ("exact", "loglin"):
            _, _, pc, pe, pre, xmax = A.attn_lowp_head(q, k, 1.0, 1.0, v, 0.6, pf, encoder=enc, return_pre=True)
            live = np.isfinite(pre)
            fmt = "e2m1" if pf == "mxfp4" else "e4m3"
            if enc == "exact":
                want = F.e2m1_encode(np.where(live, pre, 0)) if pf == "mxfp4" else F.e4m3_encode(np.where(live, pre, 0))
            else:
                want = loglin_round(pre, fmt)
            np.testing.assert_array_equal(np.where(live, want, 0), pc)
            if pf == "mxfp4":
                e = pe.astype(np.int64) - 127
                np.testing.assert_array_equal(e, np.maximum(np.floor(xmax) - 2, -127))


def test_pre_values_hand_derived():
    # x = t - m' on one tile; block 0 holds the max (x = 0 -> e = -2): pre = 2^(x + 2)
    t = np.full(32, -3.0)
    t[0], t[1] = 0.0, -1.5
    _, _, pc, pe, pre, xmax = A.attn_lowp_head(np.ones((1, 1)), t[:, None], 1.0, 1.0, np.ones((32, 1)),
                                               1.0 / A.LOG2E, "mxfp4", return_pre=True)
    np.testing.assert_allclose(pre[0, :3], [4.0, 2 ** 0.5, 0.5], rtol=1e-14)
    assert xmax[0, 0] == 0.0 and pe[0, 0] == 125


def _case(pf, enc, seed=4):
    rng = np.random.default_rng(seed)
    q, k, v = _head(rng, nq=6, nk=256)
    res = A.attn_lowp_head(q, k, 1.0, 1.0, v, 0.6, pf, encoder=enc, return_pre=True)
    return res[2].copy(), (None if res[3] is None else res[3].copy()), res[2], res[3], res[4].copy(), res[5]


@pytest.mark.parametrize("pf,enc", [("mxfp4", "exact"), ("mxfp4", "loglin"), ("fp8", "exact"), ("fp8", "loglin")])
def test_tie_check_accepts_identical_and_near_ties(pf, enc):
    gc, ge, oc, oe, pre, xmax = _case(pf, enc)
    live = np.isfinite(pre)
    assert check_code_choices(gc, ge, oc, oe, pre, xmax, pf, enc, live) == (0, 0)
    # put one live element right on a boundary and round it up instead of down
    i, j = np.argwhere(live & (oc > 1) & (oc < 6))[0]
    c = int(oc[i, j])
    if enc == "exact":
        dec = F.e2m1_decode if pf == "mxfp4" else F.e4m3_decode
        pre[i, j] = 0.5 * (dec(c) + dec(c + 1)) * (1 - 1e-7)
    else:
        pre[i, j] = c + 0.5 - 1e-5
    gc[i, j] = c + 1
    assert check_code_choices(gc, ge, oc, oe, pre, xmax, pf, enc, live) == (0, 1)


@pytest.mark.parametrize("pf,enc", [("mxfp4", "exact"), ("mxfp4", "loglin"), ("fp8", "exact"), ("fp8", "loglin")])
def test_tie_check_rejects_other_differences(pf, enc):
    gc, ge, oc, oe, pre, xmax = _case(pf, enc)
    live = np.isfinite(pre)
    i, j = np.argwhere(live & (oc > 1) & (oc < 5))[0]
    bad = gc.copy()
    bad[i, j] = oc[i, j] + 1                     # a neighbour, but not at a boundary
    lo = np.rint(pre[i, j]) if enc == "loglin" else None
    if enc == "loglin" and abs(pre[i, j] - (lo + 0.5)) < 1e-2:
        pytest.skip("drawn value sits on a boundary")
    with pytest.raises(AssertionError):
        check_code_choices(bad, ge, oc, oe, pre, xmax, pf, enc, live)
    bad = gc.copy()
    bad[i, j] = oc[i, j] + 2                     # not a neighbour
    with pytest.raises(AssertionError):
        check_code_choices(bad, ge, oc, oe, pre, xmax, pf, enc, live)


def test_tie_check_block_exponent():
    gc, ge, oc, oe, pre, xmax = _case("mxfp4", "exact", seed=5)
    live = np.isfinite(pre)
    # block 2 of row 0: claim its max sat just below an integer, so the kernel
    # took e - 1; its codes under e - 1 are the oracle's values doubled
    b = 2
    xmax = xmax.copy()
    xmax[0, b] = np.rint(xmax[0, b]) - 1e-6
    ge = ge.copy()
    ge[0, b] = oe[0, b] - 1
    keys = slice(32 * b, 32 * b + 32)
    gc[0, keys] = np.where(live[0, keys], F.e2m1_encode(np.where(live[0, keys], pre[0, keys] * 2, 0)), 0)
    n_e, _ = check_code_choices(gc, ge, oc, oe, pre, xmax, "mxfp4", "exact", live)
    assert n_e == 1
    # the same exponent change with the block max away from an integer is rejected
    xmax[0, b] = np.rint(xmax[0, b]) - 0.3
    with pytest.raises(AssertionError):
        check_code_choices(gc, ge, oc, oe, pre, xmax, "mxfp4", "exact", live)


def test_tie_check_row_slack():
    # a code rounded the other way 1e-3 (relative) from its boundary: beyond
    # the plain window, inside a row slack of 2e-3 log2 units (1.4e-3 relative)
    gc, ge, oc, oe, pre, xmax = _case("mxfp4", "exact", seed=7)
    live = np.isfinite(pre)
    i, j = np.argwhere(live & (oc > 1) & (oc < 6))[0]
    c = int(oc[i, j])
    pre[i, j] = 0.5 * (F.e2m1_decode(c) + F.e2m1_decode(c + 1)) * (1 - 1e-3)
    oc = oc.copy()
    oc[i, j] = c
    gc = gc.copy()
    gc[i, j] = c + 1
    with pytest.raises(AssertionError):
        check_code_choices(gc, ge, oc, oe, pre, xmax, "mxfp4", "exact", live)
    slack = np.zeros(gc.shape[0])
    slack[i] = 2e-3
    assert check_code_choices(gc, ge, oc, oe, pre, xmax, "mxfp4", "exact", live, row_slack=slack) == (0, 1)
    slack[i] = 1e-3                               # 0.7e-3 relative: too narrow
    with pytest.raises(AssertionError):
        check_code_choices(gc, ge, oc, oe, pre, xmax, "mxfp4", "exact", live, row_slack=slack)


def test_tie_check_row_slack_cast():
    # the E2M1 cast: a position 0.01 code units from its boundary (2^M = 2 code
    # units per log2 unit) needs a row slack of at least 0.005 - NEAR_TIE_POS / 2
    gc, ge, oc, oe, pre, xmax = _case("mxfp4", "loglin", seed=8)
    live = np.isfinite(pre)
    i, j = np.argwhere(live & (oc > 1) & (oc < 6))[0]
    c = int(oc[i, j])
    pre[i, j] = c + 0.5 - 0.01
    oc = oc.copy()
    oc[i, j] = c
    gc = gc.copy()
    gc[i, j] = c + 1
    with pytest.raises(AssertionError):
        check_code_choices(gc, ge, oc, oe, pre, xmax, "mxfp4", "loglin", live)
    slack = np.zeros(gc.shape[0])
    slack[i] = 0.005
    assert check_code_choices(gc, ge, oc, oe, pre, xmax, "mxfp4", "loglin", live, row_slack=slack) == (0, 1)
    slack[i] = 0.004
    with pytest.raises(AssertionError):
        check_code_choices(gc, ge, oc, oe, pre, xmax, "mxfp4", "loglin", live, row_slack=slack)


def test_bwd_check_zero_below_float32_normal_range():
    from helpers import check_bwd_codes
    from oracle import backward as OB
    # one block of 32 values along axis 1 whose block exponent sits at its
    # floor of -127: the value 2^-128 * 5 codes to E4M3(2.5) = 0x42 (biased
    # exponent 8, mantissa 010), but the
    # float32 probability behind it is below the normal range
    x = np.zeros((1, 32))
    x[0, :4] = [2.0 ** -120, 2.0 ** -128 * 5.0, 2.0 ** -124, -(2.0 ** -122)]
    _, oc, oe = OB.mx_e4m3(x, axis=1)
    assert int(oe[0, 0]) == -127 and int(oc[0, 1]) == 0x42
    eps = np.full(x.shape, 1e-6)
    live = np.ones(x.shape, bool)
    gc = oc.copy()
    gc[0, 1] = 0
    ge = oe + 127
    p = np.ones(x.shape)
    p[0, 1] = 2.0 ** -130
    assert check_bwd_codes(gc, ge, x, oc, ge, eps, 1, live, p=p) == 0
    # a zero code where the value and its probability are normal floats is a mismatch
    gc2 = oc.copy()
    gc2[0, 0] = 0
    with pytest.raises(AssertionError):
        check_bwd_codes(gc2, ge, x, oc, ge, eps, 1, live, p=np.ones(x.shape))
    # and a nonzero wrong code below the normal range is still rejected
    gc3 = oc.copy()
    gc3[0, 1] = 0x30
    with pytest.raises(AssertionError):
        check_bwd_codes(gc3, ge, x, oc, ge, eps, 1, live, p=p)
