"""Shared test plumbing: run the oracle and the HIP path on the same seeded
inputs and compare.  The oracle never sees anything the HIP path produced."""

import math

import numpy as np
import torch

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


# Scores far from zero: the kernel's float32 score t = c Q^.K^ (exact
# products, float32 sums on the MFMA) is within 2^-20 of c sum_d |q^_d k^_d|
# of the exact one, the bound measured for the backward's float32 scores; a
# window of SCORE_ERR_FACTOR times it is allowed on top of NEAR_* when a test
# passes it (row_slack).  Near zero the bound is far below NEAR_*.
SCORE_ERR_FACTOR = 4.0 * 2.0 ** -20


def score_row_slack(q_rows, k_rows, *, amax_q, amax_k, sigma, qk="nvfp4", four_six=False, q_index=None,
                    causal=False):
    """Per query row, in log2 units: twice the largest float32 error bound of
    its live scaled scores t = sigma log2(e) Q^.K^ (a code's y = t - m' - e
    carries the error of t and that of the running max m')."""
    if qk in ("mxfp4", "mxfp4_had"):
        had = qk == "mxfp4_had"
        qd = OQ.dequant_mxfp4(*OQ.quant_mxfp4(q_rows, hadamard=had))
        kd = OQ.dequant_mxfp4(*OQ.quant_mxfp4(k_rows, hadamard=had))
        c = sigma / 32.0 if had else sigma
    else:
        qfn = OQ.quant_nvfp4_46 if four_six else OQ.quant_nvfp4
        qc, qs, gq = qfn(q_rows, amax=amax_q)
        kc, ks, gk = qfn(k_rows, amax=amax_k)
        qd, kd = OQ.dequant_nvfp4_raw(qc, qs), OQ.dequant_nvfp4_raw(kc, ks)
        c = sigma * float(np.float32(gq)) * float(np.float32(gk))
    bound = SCORE_ERR_FACTOR * c * math.log2(math.e) * (np.abs(qd) @ np.abs(kd).T)
    if causal:
        qi = np.arange(len(q_rows)) if q_index is None else np.asarray(q_index)
        bound = np.where(np.arange(len(k_rows))[None, :] <= qi[:, None], bound, 0.0)
    return 2.0 * bound.max(axis=1)


def check_code_choices(gc, ge, oc, oe, pre, xmax, p_format, encoder, live, row_slack=None):
    """Every probability code and E8M0 block exponent in which the kernel
    differs from the oracle must be a rounding near-tie (the neighbouring
    code, the oracle's unrounded value within NEAR_* of the boundary, widened
    by row_slack [R] log2 units where given).
    gc/ge: kernel codes and exponents; oc/oe/pre/xmax: the oracle's, from
    return_pre.  Returns (differing exponents, differing element codes)."""
    fmt = "e2m1" if p_format == "mxfp4" else "e4m3"
    if row_slack is None:
        row_slack = np.zeros(gc.shape[0])
    slack = np.asarray(row_slack, np.float64)[:, None] * np.ones(gc.shape)
    R, nk = gc.shape
    pre = pre.copy()
    n_e = 0
    if p_format == "mxfp4":
        nblk = (nk + 31) // 32
        has = np.zeros((R, nblk), bool)
        for b in range(nblk):
            has[:, b] = live[:, 32 * b:32 * b + 32].any(axis=1)
        de = (ge.astype(np.int64) != oe.astype(np.int64)) & has
        n_e = int(de.sum())
        if n_e:
            bad = de & ~((np.abs(xmax - np.rint(xmax)) <= NEAR_INT + slack[:, :1])
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
        g, o, v, sl = gc[dm].astype(np.int64), oc[dm].astype(np.int64), pre[dm], slack[dm]
        adjacent = np.abs(g - o) == 1
        lo = np.minimum(g, o)
        if encoder == "exact":
            dec = OF.e2m1_decode if fmt == "e2m1" else OF.e4m3_decode
            mid = 0.5 * (dec(lo) + dec(lo + 1))
            near = np.abs(v - mid) <= (NEAR_TIE_REL + np.expm1(sl * math.log(2.0))) * mid
        else:
            # the cast position 2^M (y + b) moves 2^M code units per log2 unit
            near = np.abs(v - (lo + 0.5)) <= NEAR_TIE_POS + (2.0 if fmt == "e2m1" else 8.0) * sl
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
BWD_MISMATCH_MAX = 1e-2      # fraction of live codes that may differ (plus 2)


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
