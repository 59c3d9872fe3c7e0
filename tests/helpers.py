"""Shared test plumbing: run the oracle and the HIP path on the same seeded
inputs and compare.  The oracle never sees anything the HIP path produced."""

import math

import numpy as np

from oracle import attention as OA
from oracle import formats as OF
from oracle import quant as OQ
from oracle import loglin as OL

# Tolerances of the parity bar (float results); codes and scales are bit-exact.
P_MISMATCH_MAX = 1e-4        # fraction of live probability codes
O_REL_L2_MAX = 1e-3
O_MAX_ABS = 5e-3
LSE_REL_MAX = 1e-4           # |dLSE| <= 1e-4 * max(1, |LSE|)
# Where float32 arithmetic decides a probability code, a value on a code
# boundary may round either way.  A code that differs from the oracle's is
# accepted only when it is the neighbouring code and the oracle's unrounded
# value lies this close to the boundary between the two:
NEAR_TIE_REL = 1e-4          # exact encoders: |2^y - midpoint| / midpoint
NEAR_TIE_POS = 1e-3          # log-linear cast: |position - (c + 1/2)|, code units
NEAR_INT = 1e-4              # E8M0 block exponent: |xmax - nearest integer|


def f32(t):
    import torch    # (imported here: the oracle worker processes load this module without torch)
    return t.detach().to("cpu", torch.float32).numpy()


def rel_l2(a, b):
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def lse_err(a, b):
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    if not fin.any():
        return 0.0
    return float(np.max(np.abs(a[fin] - b[fin]) / np.maximum(1.0, np.abs(b[fin]))))


def oracle_v_head(v_head_f32, v_format, amax_all=None):
    """Dequantized V of one (sequence, kv head): [Nk, D] float64."""
    if v_format == "fp8":
        codes, s_v = OQ.quant_v_fp8(v_head_f32, amax=amax_all)
        return OQ.dequant_v_fp8(codes, s_v)
    codes, e8 = OQ.quant_v_mxfp4(v_head_f32[:, None, :])
    return OQ.dequant_v_mxfp4(codes, e8)[:, 0, :]


def oracle_head(q_rows, k_rows, v_rows, *, amax_q, amax_k, amax_v, sigma, p_format, v_format, causal,
                q_index=None, return_p=False, encoder="exact", p_given=None, return_pre=False, four_six=False,
                qk="nvfp4"):
    """Oracle forward for a set of query rows of one head, given the bf16
    inputs (as float32 numpy) and the whole-tensor amax values.  ``qk="mxfp4"``
    quantizes Q and K with the MX-native rule (E8M0 per 32 along D, no tensor
    scales) instead of NVFP4; ``qk="mxfp4_had"`` rotates each 32-element block
    by the Hadamard matrix first."""
    vh = oracle_v_head(v_rows, v_format, amax_v)
    if qk in ("mxfp4", "mxfp4_had"):
        # with the block Hadamard rotation of Q and K, every Q.K is 32 times the
        # original, so the forward runs with sigma / 32
        had = qk == "mxfp4_had"
        qc, qe = OQ.quant_mxfp4(q_rows, hadamard=had)
        kc, ke = OQ.quant_mxfp4(k_rows, hadamard=had)
        sigma = sigma / 32.0 if had else sigma
        return OA.attn_lowp_head(OQ.dequant_mxfp4(qc, qe), OQ.dequant_mxfp4(kc, ke), 1.0, 1.0, vh, sigma,
                                 p_format, causal, q_index=q_index, return_p=return_p, encoder=encoder,
                                 p_given=p_given, return_pre=return_pre)
    qfn = OQ.quant_nvfp4_46 if four_six else OQ.quant_nvfp4
    qc, qs, gq = qfn(q_rows, amax=amax_q)
    kc, ks, gk = qfn(k_rows, amax=amax_k)
    return OA.attn_lowp_head(OQ.dequant_nvfp4_raw(qc, qs), OQ.dequant_nvfp4_raw(kc, ks), gq, gk, vh, sigma,
                             p_format, causal, q_index=q_index, return_p=return_p, encoder=encoder,
                             p_given=p_given, return_pre=return_pre)


def p_mismatch(gpu_codes, gpu_scales, ora_codes, ora_e8, p_format, nk, live):
    """Count probability codes whose dequantized value differs (a differing
    block scale counts for every live key of the block).  gpu_codes is the
    debug dump (packed nibbles for MXFP4), ora_* from the oracle."""
    if p_format == "mxfp4":
        gc = OF.unpack_nibbles(gpu_codes)[:, :nk]
        gv = OF.e2m1_decode(gc) * np.repeat(OF.e8m0_decode(gpu_scales), 32, axis=1)[:, :nk]
        ov = OF.e2m1_decode(ora_codes) * np.repeat(OF.e8m0_decode(ora_e8), 32, axis=1)[:, :nk]
    else:
        gv = OF.e4m3_decode(gpu_codes[:, :nk])
        ov = OF.e4m3_decode(ora_codes)
    diff = (gv != ov) & live
    return int(diff.sum()), int(live.sum())


def assert_close_outputs(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    r = rel_l2(o_gpu, o_ref)
    ma = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    le = lse_err(lse_gpu, lse_ref)
    assert r <= O_REL_L2_MAX, f"{what}: O rel L2 {r:.3e}"
    assert ma <= O_MAX_ABS, f"{what}: O max abs {ma:.3e}"
    assert le <= LSE_REL_MAX, f"{what}: LSE rel {le:.3e}"
    return r, ma, le


def gpu_codes(dump_codes, dump_scales, p_format, nk):
    """Debug dump rows -> (codes [R, nk] in key order, E8M0 bytes [R, ceil(nk/32)] or None)."""
    if p_format == "mxfp4":
        return OF.unpack_nibbles(dump_codes)[:, :nk], dump_scales[:, :(nk + 31) // 32]
    return dump_codes[:, :nk], None


def check_code_choices(gc, ge, oc, oe, pre, xmax, p_format, encoder, live):
    """Every probability code and E8M0 block exponent in which the kernel
    differs from the oracle must be a rounding near-tie (the neighbouring
    code, the oracle's unrounded value within NEAR_* of the boundary).
    gc/ge: kernel codes and exponents; oc/oe/pre/xmax: the oracle's, from
    return_pre.  Returns (differing exponents, differing element codes)."""
    fmt = "e2m1" if p_format == "mxfp4" else "e4m3"
    R, nk = gc.shape
    pre = pre.copy()
    n_e = 0
    if p_format == "mxfp4":
        nblk = (nk + 31) // 32
        has = np.pad(live, ((0, 0), (0, 32 * nblk - nk))).reshape(R, nblk, 32).any(axis=2)
        de = (ge.astype(np.int64) != oe.astype(np.int64)) & has
        n_e = int(de.sum())
        if n_e:
            bad = de & ~((np.abs(xmax - np.rint(xmax)) <= NEAR_INT)
                         & (np.abs(ge.astype(np.int64) - oe.astype(np.int64)) == 1))
            assert not bad.any(), f"E8M0 exponents differ away from a boundary at {np.argwhere(bad)[:5].tolist()}"
        # the oracle's unrounded values under the kernel's exponents
        shift = np.repeat(oe.astype(np.int64) - ge.astype(np.int64), 32, axis=1)[:, :nk]
        fin = np.isfinite(pre)
        if encoder == "exact":
            pre[fin] = pre[fin] * np.exp2(shift[fin])
        else:
            pre[fin] = pre[fin] + 2.0 * shift[fin]
        if encoder == "exact":
            oc = np.where(live, OF.e2m1_encode(np.where(fin, pre, 0.0)), 0).astype(np.uint8)
        else:
            oc = np.where(live, OL.loglin_round(pre, fmt), 0).astype(np.uint8)
    dm = (gc.astype(np.int64) != oc.astype(np.int64)) & live
    n_c = int(dm.sum())
    if n_c:
        g, o, v = gc[dm].astype(np.int64), oc[dm].astype(np.int64), pre[dm]
        adjacent = np.abs(g - o) == 1
        lo = np.minimum(g, o)
        if encoder == "exact":
            dec = OF.e2m1_decode if fmt == "e2m1" else OF.e4m3_decode
            mid = 0.5 * (dec(lo) + dec(lo + 1))
            near = np.abs(v - mid) <= NEAR_TIE_REL * mid
        else:
            # the cast position 2^M (y + b) moves 2^M code units per log2 unit
            near = np.abs(v - (lo + 0.5)) <= NEAR_TIE_POS
        bad = ~(adjacent & near)
        where = np.argwhere(dm)[bad][:5].tolist()
        assert not bad.any(), (f"{int(bad.sum())} codes differ away from a rounding boundary, e.g. at {where}: "
                               f"kernel {g[bad][:5].tolist()} oracle {o[bad][:5].tolist()} value {v[bad][:5].tolist()}")
    return n_e, n_c


# ---- backward: E4M3 operands decided in float32 --------------------------
# The kernel computes P = 2^(t - L) and dS = P (dP - D) in float32.  Error
# sources, each bounded by a multiple of the sum of the magnitudes of its
# terms (measured on gfx950):
#  * t = c Q.K on the bf16 MFMA: products exact, sums keep 24 bits below the
#    largest product -> 2^-20 of |c| sum |Q||K|;
#  * dP = dO^.V^ on the FP8 MFMA: each group of 8 products is aligned to its
#    largest product and truncated 15 bits below it -> 2^-11 of sum |dO^||V^|;
#  * D: a float32 sum over D terms -> 2^-20 of sum |dO^ O|;
# and dP - D cancels, which divides by |dP - D|.  A code that differs from
# the oracle's is accepted when it is the E4M3 rounding of some value within
# BWD_TIE_FACTOR times that bound of the exact value.
BWD_TIE_FACTOR = 4.0
BWD_MISMATCH_MAX = 1e-3      # fraction of live codes that may differ (plus 2)


def _bwd_rel_err(abs_t, lse2, ds=None, p=None, abs_dpv=None, abs_D=None):
    """Relative float32 error bound of P (and of dS when ds is given)."""
    eps = math.log(2.0) * 2.0 ** -20 * (abs_t + np.abs(lse2)) + 2.0 ** -20
    if ds is not None:
        with np.errstate(divide="ignore", invalid="ignore"):
            diff = np.where(p > 0, np.abs(ds) / np.where(p > 0, p, 1.0), np.inf)
            eps = eps + (2.0 ** -11 * abs_dpv + 2.0 ** -20 * abs_D) / diff + 2.0 ** -20
    return eps


F32_MIN_NORMAL = 2.0 ** -126


def check_bwd_codes(gc, ge, x, oc, oe, eps, axis, live, what="", p=None):
    """Kernel E4M3 codes gc with E8M0 bytes ge (blocks of 32 along ``axis``)
    against the oracle's (oc, oe) for exact values x with relative error
    bounds eps.  Exponents may differ only where the block max is within its
    error of a power of two; codes only at rounding near-ties.  With the
    exact probabilities p: where p or x lies below the float32 normal range,
    the kernel's exponential (which returns no subnormal) or its float32
    product is 0, so a kernel code of 0 is accepted there (a block exponent at
    its floor of -127 scales such values into the E4M3 range).  Returns the
    number of differing live codes (those zero codes not counted)."""
    gc = np.asarray(gc); oc = np.asarray(oc)
    rep = lambda e: np.repeat(np.asarray(e, np.int64), 32, axis=axis)[:x.shape[0], :x.shape[1]]
    eg, eo = rep(ge) - 127, rep(oe) - 127
    de = (eg != eo) & live
    if de.any():
        # the block's largest magnitude must sit on the power of two that separates the exponents
        amax = np.abs(x)
        lim = np.ldexp(1.0, np.maximum(eg, eo) + 8)
        ok = (np.abs(eg - eo) == 1) & (np.abs(amax - lim) <= BWD_TIE_FACTOR * eps * lim)
        blk_ok = np.zeros_like(de)
        # a block passes if some live element of it is that near-boundary maximum
        n = x.shape[axis]
        for b0 in range(0, n, 32):
            sl = (slice(b0, b0 + 32), slice(None)) if axis == 0 else (slice(None), slice(b0, b0 + 32))
            any_ok = (ok[sl] & live[sl]).any(axis=axis, keepdims=True)
            blk_ok[sl] = np.broadcast_to(any_ok, blk_ok[sl].shape)
        bad = de & ~blk_ok
        assert not bad.any(), f"{what}: E8M0 exponents differ away from a boundary at {np.argwhere(bad)[:4].tolist()}"
    y = x * np.exp2(-eg.astype(np.float64))
    ref = np.where(live, OF.e4m3_encode(np.clip(np.where(live, y, 0.0), -448, 448)), 0)
    gval, rval = OF.e4m3_decode(gc), OF.e4m3_decode(ref)
    diff = (gval != rval) & live
    if p is not None:
        below = (np.asarray(p) < F32_MIN_NORMAL) | (np.abs(x) < F32_MIN_NORMAL)
        diff &= ~(below & (gval == 0))
    n_diff = int(diff.sum())
    if n_diff:
        # the kernel's code must be the rounding of some value within the error
        # bound of the exact one: rounding is monotone, so its value must lie
        # between the roundings of the interval's ends
        half = BWD_TIE_FACTOR * np.where(np.isfinite(eps), eps, 1e30) * np.abs(y)
        ends = [OF.e4m3_decode(OF.e4m3_encode(np.clip(np.where(live, y + sgn * half, 0.0), -448, 448)))
                for sgn in (-1.0, 1.0)]
        near = (gval >= np.minimum(*ends)) & (gval <= np.maximum(*ends))
        bad = diff & ~near
        where = np.argwhere(bad)[:4].tolist()
        assert not bad.any(), (f"{what}: {int(bad.sum())} E4M3 codes lie outside the rounding of the float32 error "
                               f"interval, e.g. at {where}: kernel {gc[bad][:4].tolist()} oracle "
                               f"{ref[bad][:4].tolist()} scaled value {y[bad][:4].tolist()} relative error bound "
                               f"{eps[bad][:4].tolist()}")
    assert n_diff <= BWD_MISMATCH_MAX * int(live.sum()) + 2, f"{what}: {n_diff} of {int(live.sum())} codes differ"
    return n_diff


# ---- forward: comparison with the oracle's own outputs --------------------
# The kernel's O and LSE are compared with the oracle's, never with the oracle
# run on the kernel's codes.  A probability code or block exponent that sits
# on a rounding boundary (within NEAR_* of it, as check_code_choices accepts)
# may legitimately come out as its neighbour in float32; on each row the bars
# are widened by the most that ALL of the oracle's own near-tie candidates,
# flipped together, could move that row's O and LSE.  The bound is computed
# from oracle quantities alone (its unrounded values, codes, block exponents,
# per-tile running maxima, l and V^), so it does not depend on which ties the
# kernel happened to take.  Rows without candidates keep the plain bars.

def oracle_prepare_kv(k_rows, v_rows, *, amax_k, amax_v, v_format, four_six=False, qk="nvfp4"):
    """The oracle's K (exact values without tensor scale, and that scale) and
    dequantized V of one (sequence, KV head): (k_raw, gk, v_hat)."""
    vh = oracle_v_head(v_rows, v_format, amax_v)
    if qk in ("mxfp4", "mxfp4_had"):
        kc, ke = OQ.quant_mxfp4(k_rows, hadamard=qk == "mxfp4_had")
        return OQ.dequant_mxfp4(kc, ke), 1.0, vh
    kc, ks, gk = (OQ.quant_nvfp4_46 if four_six else OQ.quant_nvfp4)(k_rows, amax=amax_k)
    return OQ.dequant_nvfp4_raw(kc, ks), gk, vh


def oracle_prepare_q(q_rows, *, amax_q, sigma, four_six=False, qk="nvfp4"):
    """The oracle's Q rows (exact values without tensor scale), that scale,
    and the softmax scale the forward runs with: (q_raw, gq, sigma_eff)."""
    if qk in ("mxfp4", "mxfp4_had"):
        had = qk == "mxfp4_had"
        qc, qe = OQ.quant_mxfp4(q_rows, hadamard=had)
        # rotated Q.K is 32 times the original
        return OQ.dequant_mxfp4(qc, qe), 1.0, (sigma / 32.0 if had else sigma)
    qc, qs, gq = (OQ.quant_nvfp4_46 if four_six else OQ.quant_nvfp4)(q_rows, amax=amax_q)
    return OQ.dequant_nvfp4_raw(qc, qs), gq, sigma


def oracle_prepare_head(q_rows, k_rows, v_rows, *, amax_q, amax_k, amax_v, sigma, v_format, four_six=False,
                        qk="nvfp4"):
    """Quantize one (sequence, head) once for the oracle: returns
    (q_raw, k_raw, gq, gk, v_hat, sigma_eff), the arguments of
    OA.attn_lowp_head, so that row chunks can run without requantizing."""
    vh = oracle_v_head(v_rows, v_format, amax_v)
    if qk in ("mxfp4", "mxfp4_had"):
        had = qk == "mxfp4_had"
        qc, qe = OQ.quant_mxfp4(q_rows, hadamard=had)
        kc, ke = OQ.quant_mxfp4(k_rows, hadamard=had)
        return OQ.dequant_mxfp4(qc, qe), OQ.dequant_mxfp4(kc, ke), 1.0, 1.0, vh, (sigma / 32.0 if had else sigma)
    qfn = OQ.quant_nvfp4_46 if four_six else OQ.quant_nvfp4
    qc, qs, gq = qfn(q_rows, amax=amax_q)
    kc, ks, gk = qfn(k_rows, amax=amax_k)
    return OQ.dequant_nvfp4_raw(qc, qs), OQ.dequant_nvfp4_raw(kc, ks), gq, gk, vh, sigma


def _tie_steps(pre, codes, fmt, encoder):
    """Per element: the largest change of the decoded value (in units of the
    element's own scale) that one near-tie rounding could make -- the gap to
    the neighbouring code across a boundary the unrounded value lies within
    NEAR_* of -- and 0 away from boundaries or where masked."""
    dec = OF.e2m1_decode if fmt == "e2m1" else OF.e4m3_decode
    top = 7 if fmt == "e2m1" else 0x7E
    c = codes.astype(np.int64)
    v, up, dn = dec(c), dec(np.minimum(c + 1, top)), dec(np.maximum(c - 1, 0))
    fin = np.isfinite(pre)
    x = np.where(fin, pre, -1.0)
    if encoder == "exact":
        mu, md = 0.5 * (v + up), 0.5 * (v + dn)
        near_up = (c < top) & (np.abs(x - mu) <= NEAR_TIE_REL * mu)
        near_dn = (c > 0) & (np.abs(x - md) <= NEAR_TIE_REL * md)
    else:
        near_up = (c < top) & (np.abs(x - (c + 0.5)) <= NEAR_TIE_POS)
        near_dn = (c > 0) & (np.abs(x - (c - 0.5)) <= NEAR_TIE_POS)
    step = np.maximum(np.where(near_up, up - v, 0.0), np.where(near_dn, v - dn, 0.0))
    return np.where(fin, step, 0.0)


def tie_flip_bound(pre, codes, e8, xmax, tiles, O, v_hat, p_format, encoder, live):
    """Oracle-only bound of how far O ([R, D], elementwise) and LSE ([R])
    of each row can move when any subset of the oracle's near-tie element
    codes and E8M0 block exponents is decided the other way.

    With d_j >= 0 the largest change of key j's dequantized probability,
    carried to the final scale by 2^(m'_tile(j) - m), S = sum_j d_j, and the
    final l:  O' - O = sum_j delta_j (V^_j - O) / (l + sum_j delta_j), so
    |O' - O| <= (sum_j d_j |V^_j| + S |O|) / (l - S), and
    |LSE' - LSE| <= -ln(1 - S / l).  Returns (o_bound, lse_bound, S / l)."""
    fmt = "e2m1" if p_format == "mxfp4" else "e4m3"
    R, nk = pre.shape
    step = _tie_steps(pre, codes, fmt, encoder)
    if p_format == "mxfp4":
        e = np.repeat(e8.astype(np.int64) - 127, 32, axis=1)[:, :nk]
        d = step * np.exp2(e)
        # block exponents whose block max lies within NEAR_INT of an integer:
        # just below n the oracle has floor n - 1 and the kernel may take n
        # (e + 1); at or just above n the kernel may take n - 1 (e - 1)
        xm = np.where(np.isfinite(xmax), xmax, 0.0)
        n = np.rint(xm)
        cand = np.isfinite(xmax) & (np.abs(xm - n) <= NEAR_INT)
        # The block holding the running max has xmax = 0 exactly on both sides
        # (x = t - m' is 0 at the max element); it can only move if another
        # key of the same tile lies within NEAR_INT of that max, so that the
        # float32 max may be taken at a different key.
        with np.errstate(divide="ignore", invalid="ignore"):
            x = (np.log2(np.where(np.isfinite(pre), pre, 0.0)) if encoder == "exact"
                 else np.where(np.isfinite(pre), pre, -np.inf) / 2.0 - 1.0) + e
        close = np.where(live, x >= -NEAR_INT, False)
        ntile = (nk + 127) // 128
        per_tile = np.pad(close, ((0, 0), (0, 128 * ntile - nk))).reshape(R, ntile, 128).sum(axis=2)
        nblk = xmax.shape[1]
        rival = np.repeat(per_tile >= 2, 4, axis=1)[:, :nblk]
        cand &= (xm != 0.0) | rival
        if cand.any():
            ealt = np.where(xm < n, 1, -1) + (e8.astype(np.int64) - 127)
            ealt = np.maximum(ealt, -127)
            cand &= ealt != (e8.astype(np.int64) - 127)
            for r, b in np.argwhere(cand):
                k0, k1 = 32 * b, min(32 * b + 32, nk)
                eo, ea = int(e8[r, b]) - 127, int(ealt[r, b])
                pr = pre[r, k0:k1]
                fin = np.isfinite(pr)
                if encoder == "exact":
                    p2 = np.where(fin, pr * 2.0 ** (eo - ea), 0.0)
                    c2 = OF.e2m1_encode(p2)
                else:
                    p2 = np.where(fin, pr + 2.0 * (eo - ea), -1.0)
                    c2 = OL.loglin_round(p2, "e2m1")
                c2 = np.where(fin, c2, 0)
                moved = np.abs(OF.e2m1_decode(c2) * 2.0 ** ea - OF.e2m1_decode(codes[r, k0:k1]) * 2.0 ** eo)
                moved += _tie_steps(np.where(fin, p2, -np.inf)[None], c2[None], "e2m1", encoder)[0] * 2.0 ** ea
                d[r, k0:k1] += np.where(fin, moved, 0.0)
    else:
        d = step
    d = np.where(live, d, 0.0)
    tile = np.arange(nk) // 128
    with np.errstate(invalid="ignore", over="ignore"):
        w = np.exp2(tiles["m_tile"][:, tile] - tiles["m"][:, None])
    w = np.where(np.isfinite(w), w, 0.0)
    d = d * w
    S = d.sum(axis=1)
    l = tiles["l"]
    frac = np.where(l > 0, S / np.where(l > 0, l, 1.0), 0.0)
    ok = frac < 1.0
    den = np.where(ok, l - S, 1.0)
    ob = (d @ np.abs(v_hat) + S[:, None] * np.abs(O)) / den[:, None]
    # past S >= l a row's O can be anything in the hull of the V^ rows
    ob = np.where(ok[:, None], ob, 2.0 * np.abs(v_hat).max(initial=0.0))
    with np.errstate(divide="ignore"):
        lb = np.where(ok, -np.log1p(-np.minimum(frac, 0.999999)), np.inf)
    return ob, lb, frac


class PureCompare:
    """Accumulates the comparison of kernel outputs with the oracle's own O
    and LSE over many row chunks: elementwise max abs <= O_MAX_ABS + o_bound,
    |dLSE| <= LSE_REL_MAX max(1, |LSE|) + lse_bound, and at the end the
    relative L2 of the whole compared tensor <= O_REL_L2_MAX plus the L2 of
    the bound relative to the oracle's norm.  Also counts the rows that
    needed the widening (error past the plain bar, within the widened one)."""

    def __init__(self, what):
        self.what = what
        self.err2 = self.ref2 = self.bnd2 = 0.0
        self.max_abs = self.lse_rel = 0.0
        self.rows = self.rows_widened = self.rows_with_ties = 0

    def add(self, o_gpu, lse_gpu, O, L, o_bound=None, lse_bound=None):
        o_gpu = np.asarray(o_gpu, np.float64)
        if o_bound is None:
            o_bound = np.zeros_like(O)
            lse_bound = np.zeros(O.shape[0])
        diff = np.abs(o_gpu - O)
        fin_b = np.isfinite(o_bound)
        self.err2 += float((diff ** 2).sum())
        self.ref2 += float((O ** 2).sum())
        self.bnd2 += float((np.where(fin_b, o_bound, 0.0) ** 2).sum())
        bad = diff > O_MAX_ABS + o_bound
        assert not bad.any(), (f"{self.what}: O differs from the oracle by {diff[bad][:4].tolist()} at "
                               f"{np.argwhere(bad)[:4].tolist()} (bound {o_bound[bad][:4].tolist()})")
        fin = np.isfinite(L)
        assert np.array_equal(np.isfinite(lse_gpu), fin), f"{self.what}: LSE finiteness differs"
        dl = np.where(fin, np.abs(np.where(fin, lse_gpu, 0.0) - np.where(fin, L, 0.0)), 0.0)
        tol = LSE_REL_MAX * np.maximum(1.0, np.abs(np.where(fin, L, 0.0)))
        badl = dl > tol + lse_bound
        assert not badl.any(), (f"{self.what}: LSE differs from the oracle by {dl[badl][:4].tolist()} at rows "
                                f"{np.argwhere(badl)[:4].ravel().tolist()} (bound {lse_bound[badl][:4].tolist()})")
        row_over = (diff > O_MAX_ABS).any(axis=1) | (dl > tol)
        self.rows += O.shape[0]
        self.rows_widened += int(row_over.sum())
        self.rows_with_ties += int(((o_bound > 0).any(axis=1) | (lse_bound > 0)).sum())
        self.max_abs = max(self.max_abs, float(diff.max(initial=0.0)))
        self.lse_rel = max(self.lse_rel, float((dl / np.maximum(1.0, np.abs(np.where(fin, L, 0.0)))).max(initial=0.0)))

    def finish(self):
        ref = math.sqrt(self.ref2) if self.ref2 > 0 else 1.0
        rel = math.sqrt(self.err2) / ref
        allow = O_REL_L2_MAX + math.sqrt(self.bnd2) / ref
        assert rel <= allow, f"{self.what}: O rel L2 {rel:.3e} against the oracle (allowed {allow:.3e})"
        return rel


# ---- backward: comparison with the oracle's own gradients -----------------

def bwd_flip_delta(gc_like_codes, exps, x, eps, axis, live, p=None):
    """Oracle-only bound, per element, of how far the kernel's dequantized
    MX E4M3 operand can lie from the oracle's where check_bwd_codes would
    accept a different code or block exponent: the rounding of the float32
    error interval of the exact value x (half-width BWD_TIE_FACTOR * eps *
    |y| in scaled units y = x 2^-e), the other exponent for blocks whose
    largest magnitude sits within that error of a power of two, and the
    zero code where p or x is below the float32 normal range."""
    codes = np.asarray(gc_like_codes)
    n0, n1 = x.shape
    rep = lambda e: np.repeat(np.asarray(e, np.int64), 32, axis=axis)[:n0, :n1]
    e = rep(exps) - 127
    cur = OF.e4m3_decode(codes) * np.exp2(e.astype(np.float64))
    y = x * np.exp2(-e.astype(np.float64))
    epsf = np.where(np.isfinite(eps), eps, 1e30)
    half = BWD_TIE_FACTOR * epsf * np.abs(y)
    d = np.zeros_like(x)
    for sgn in (-1.0, 1.0):
        end = OF.e4m3_decode(OF.e4m3_encode(np.clip(np.where(live, y + sgn * half, 0.0), -448, 448)))
        d = np.maximum(d, np.abs(end * np.exp2(e.astype(np.float64)) - cur))
    # block exponents: the kernel may sit one binade off where the block's
    # largest magnitude is within its error bound of 2^(e+8) or 2^(e+9)
    amax = np.abs(x)
    for de in (-1, 1):
        lim = np.exp2((e + (8 if de < 0 else 9)).astype(np.float64))
        near = live & (np.abs(amax - lim) <= BWD_TIE_FACTOR * epsf * lim)
        blk = np.zeros_like(near)
        for b0 in range(0, x.shape[axis], 32):
            sl = (slice(b0, b0 + 32), slice(None)) if axis == 0 else (slice(None), slice(b0, b0 + 32))
            blk[sl] = np.broadcast_to(near[sl].any(axis=axis, keepdims=True), blk[sl].shape)
        if blk.any():
            ea = (e + de).astype(np.float64)
            alt = OF.e4m3_decode(OF.e4m3_encode(np.clip(np.where(live, x * np.exp2(-ea), 0.0), -448, 448)))
            d = np.maximum(d, np.where(blk, np.abs(alt * np.exp2(ea) - cur) + 2.0 ** -3 * np.abs(x), 0.0))
    if p is not None:
        below = (np.asarray(p) < F32_MIN_NORMAL) | (np.abs(x) < F32_MIN_NORMAL)
        d = np.maximum(d, np.where(below, np.abs(cur), 0.0))
    return np.where(live, d, 0.0)
