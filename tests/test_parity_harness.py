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


# ---- the oracle-only bounds that widen the pure-oracle comparison ---------

def _perturbed_codes(pf, enc, pre, xmax, oe, live, rng, tol_rel, tol_pos, tol_int):
    """Codes a float32 implementation could produce: every unrounded value
    moved by up to 0.9 of its near-tie window, every block max by up to 0.9
    of NEAR_INT, then rounded again."""
    fmt = "e2m1" if pf == "mxfp4" else "e4m3"
    nq, nk = pre.shape
    ge = None
    shift = np.zeros((nq, nk))
    if pf == "mxfp4":
        # (a block whose max is the running max has xmax = 0 exactly on both sides)
        xm = np.where(xmax == 0.0, 0.0, xmax + rng.uniform(-0.9, 0.9, xmax.shape) * tol_int)
        e_new = np.where(np.isfinite(xmax), np.maximum(np.floor(np.where(np.isfinite(xm), xm, 0.0)) - 2, -127),
                         oe.astype(np.int64) - 127)
        ge = (e_new + 127).astype(np.uint8)
        shift = np.repeat(oe.astype(np.int64) - 127 - e_new, 32, axis=1)[:, :nk]
    fin = np.isfinite(pre)
    u = rng.uniform(-0.9, 0.9, pre.shape)
    if enc == "exact":
        x = np.where(fin, pre * np.exp2(shift) * (1 + u * tol_rel), 0.0)
        gc = F.e2m1_encode(x) if fmt == "e2m1" else F.e4m3_encode(x)
    else:
        x = np.where(fin, pre + (2.0 if fmt == "e2m1" else 8.0) * shift + u * tol_pos, -1.0)
        gc = loglin_round(x, fmt)
    return np.where(live, gc, 0).astype(np.uint8), ge


@pytest.mark.parametrize("pf,enc", [("mxfp4", "exact"), ("mxfp4", "loglin"), ("fp8", "exact"), ("fp8", "loglin")])
def test_tie_bound_covers_every_near_tie_rounding(monkeypatch, pf, enc):
    import helpers
    tol_rel, tol_pos, tol_int = 0.02, 0.05, 0.05      # wide windows: many candidates per row
    monkeypatch.setattr(helpers, "NEAR_TIE_REL", tol_rel)
    monkeypatch.setattr(helpers, "NEAR_TIE_POS", tol_pos)
    monkeypatch.setattr(helpers, "NEAR_INT", tol_int)
    rng = np.random.default_rng(11)
    q, k, v = _head(rng, nq=10, nk=333, d=16)
    qi = np.arange(10) * 33 + 20
    for causal in (False, True):
        res = A.attn_lowp_head(q, k, 1.0, 1.0, v, 0.7, pf, causal=causal, q_index=qi, encoder=enc,
                               return_pre=True, return_tiles=True)
        O, L, oc, oe, pre, xmax, tiles = res
        live = np.isfinite(pre)
        ob, lb, frac = helpers.tie_flip_bound(pre, oc, oe, xmax, tiles, O, v, pf, enc, live)
        assert (ob > 0).any() and (frac < 0.5).all()
        moved = 0.0
        for trial in range(12):
            gc, ge = _perturbed_codes(pf, enc, pre, xmax, oe, live, rng, tol_rel, tol_pos, tol_int)
            O2, L2 = A.attn_lowp_head(q, k, 1.0, 1.0, v, 0.7, pf, causal=causal, q_index=qi, encoder=enc,
                                      p_given=(gc, ge))
            assert (np.abs(O2 - O) <= ob + 1e-12).all()
            assert (np.abs(L2 - L) <= lb + 1e-12).all()
            moved = max(moved, float(np.abs(O2 - O).max()))
        assert moved > 0, "no perturbed rounding changed any code: the test is vacuous"


def test_tie_bound_zero_without_candidates():
    import helpers
    rng = np.random.default_rng(12)
    q, k, v = _head(rng, nq=4, nk=200, d=16)
    res = A.attn_lowp_head(q, k, 1.0, 1.0, v, 0.7, "mxfp4", return_pre=True, return_tiles=True)
    O, L, oc, oe, pre, xmax, tiles = res
    # no unrounded value lies within the (tiny) default windows of a boundary here
    ob, lb, frac = helpers.tie_flip_bound(pre, oc, oe, xmax, tiles, O, v, "mxfp4", "exact", np.isfinite(pre))
    assert not ob.any() and not lb.any()


def test_pure_compare_bars():
    from helpers import PureCompare, O_MAX_ABS
    O = np.ones((3, 4))
    L = np.array([1.0, 2.0, -np.inf])
    pc = PureCompare("t")
    pc.add(O + 0.5 * O_MAX_ABS, L, O, L)
    with pytest.raises(AssertionError):
        PureCompare("t").add(O + 2 * O_MAX_ABS, L, O, L)
    # the widened bound admits the same error on a row with candidates
    ob = np.zeros_like(O)
    ob[1] = 2 * O_MAX_ABS
    pc2 = PureCompare("t")
    pc2.add(O + np.array([[0.0], [2.5 * O_MAX_ABS], [0.0]]), L, O, L, ob, np.zeros(3))
    assert pc2.rows_widened == 1
    with pytest.raises(AssertionError):
        PureCompare("t").add(O, L + np.array([0.0, 1e-3, 0.0]), O, L)


def test_bwd_flip_bound_covers_perturbed_operands():
    from helpers import BWD_TIE_FACTOR, bwd_flip_delta
    from oracle import backward as OB
    rng = np.random.default_rng(13)
    N, D = 70, 16
    q = rng.standard_normal((N, D))
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, D))
    o = rng.standard_normal((N, D)) * 0.3
    do = rng.standard_normal((N, D))
    lse = np.log(np.exp(0.5 * q @ k.T * np.tril(np.ones((N, N)))).sum(1))
    args = (q, k, 1.0, 1.0, v, o, do, lse, 0.5, True)
    dq, dk, dv, pre = OB.attn_bwd_head(*args, return_pre=True)
    eps = 3e-3                                            # a wide error bound: many candidates
    pq, pk = pre["q"], pre["k"]
    live_q, live_k = pq["p"] > 0, pk["p"] > 0
    e_q = np.full(pq["ds"].shape, eps)
    e_k = np.full(pk["p"].shape, eps)
    d_dsq = bwd_flip_delta(pq["codes"], pq["exps"], pq["ds"], e_q, 1, live_q)
    d_pt = bwd_flip_delta(pk["codes_p"], pk["exps_p"], pk["p"], e_k, 0, live_k)
    d_dsk = bwd_flip_delta(pk["codes_ds"], pk["exps_ds"], pk["ds"], e_k, 0, live_k)
    b_dq = 0.5 * d_dsq @ np.abs(k)
    b_dv = d_pt.T @ np.abs(do)
    b_dk = 0.5 * d_dsk.T @ np.abs(q)
    moved = 0.0
    for trial in range(10):
        # operands a float32 implementation could round: each exact value moved
        # by up to 0.9 of BWD_TIE_FACTOR times its error bound, then MX-quantized
        pert = lambda x: x * (1 + rng.uniform(-0.9, 0.9, x.shape) * BWD_TIE_FACTOR * eps)
        _, cq, eq = OB.mx_e4m3(pert(pq["ds"]), axis=1)
        _, cp, ep = OB.mx_e4m3(pert(pk["p"]), axis=0)
        _, ck, ek = OB.mx_e4m3(pert(pk["ds"]), axis=0)
        g = {"ds_q": (cq, eq + 127), "p_t": (cp, ep + 127), "ds_k": (ck, ek + 127)}
        dq2, dk2, dv2 = OB.attn_bwd_head(*args, given=g)
        assert (np.abs(dq2 - dq) <= b_dq + 1e-12).all()
        assert (np.abs(dv2 - dv) <= b_dv + 1e-12).all()
        assert (np.abs(dk2 - dk) <= b_dk + 1e-12).all()
        moved = max(moved, float(np.abs(dv2 - dv).max()))
    assert moved > 0
