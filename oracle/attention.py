"""Tiled low-precision attention forward of the oracle.  TEST INFRASTRUCTURE ONLY.

Follows "Hardware-Aware FP4 FlashAttention-4" (summary page, "What the paper
found", and the abstract on the arXiv listing 2609.04105v1): Q and K stay
NVFP4; the row-max-shifted log2 scores are mapped straight to MXFP4 E2M1
probability codes; the denominator is summed from the same rounded
probabilities that the P.V product consumes; the FP8 P/V variant keeps
E4M3 probabilities and values.  Steps the pages leave open, and the reading
taken for each:

* Tiling of the online softmax: the running max is updated once per tile of
  128 consecutive keys aligned to key 0, every tile, with no skipped rescale.
* P blocks: 32 consecutive keys aligned to the tile (hence to key 0).
* P block scale: the OCP MX rule on the block's largest probability,
  e = max(floor(xmax) - 2, -127) with xmax the block max of t - m'; a block
  with no live key gets e = -127 and zero codes.
* FP8 P uses a unit scale: code = E4M3(2**(t - m')).
* ``encoder="loglin"`` swaps the element map for the exp-free log-linear
  cast of the related pages (VC-Attention for E4M3, EFQ-Softmax for block
  E2M1; see ``oracle.loglin``): same running max, same block exponent e,
  code = loglin(t - m' - e) instead of RNE(2**(t - m' - e)).
* Masked (causal: key > query; or past the end) keys contribute nothing.
* LSE is the natural log built from the quantized denominator:
  LSE = ln2 * (m + log2 l).  A row with no live key gives O = 0, LSE = -inf.

All attention arithmetic is float64.  The raw score Q_raw . K_raw is exact in
float64 (every product of two NVFP4 values without tensor scale needs at most
12 significant bits); the tensor scales, the softmax scale and log2(e) are
folded into one float64 constant c, so t = c * S_raw.
"""

import math

import numpy as np

from .formats import e2m1_encode, e2m1_decode, e4m3_encode, e4m3_decode
from .loglin import loglin_encode, loglin_position

TILE = 128
PBLOCK = 32
LOG2E = 1.0 / math.log(2.0)
LN2 = math.log(2.0)


def attn_lowp_head(q_raw, k_raw, gq, gk, v_hat, sigma, p_format="mxfp4",
                   causal=False, q_index=None, return_p=False, encoder="exact",
                   p_given=None, return_pre=False, return_tiles=False):
    """One (batch, head): tiled Direct-P (``p_format="mxfp4"``) or FP8-P
    (``p_format="fp8"``) forward.

    q_raw  float64 [nq, D]  E2M1 * E4M3 block scale (no tensor scale)
    k_raw  float64 [Nk, D]  same for K
    gq, gk                  FP32 tensor scales of Q and K
    v_hat  float64 [Nk, Dv] fully dequantized V
    sigma                   softmax scale
    q_index int [nq]        absolute query positions (for the causal mask);
                            defaults to 0..nq-1
    encoder                 "exact" (RNE of 2**y) or "loglin" (exp-free cast)
    Returns (O [nq, Dv], LSE [nq]) and, with ``return_p``, the probability
    codes [nq, Nk] (uint8, 0 where masked) and, for MXFP4, the E8M0 bytes
    [nq, ceil(Nk/32)].

    Two hooks for checking an implementation whose float32 arithmetic may
    round a value that lies on a code boundary the other way:
    p_given     (codes [nq, Nk], E8M0 bytes [nq, ceil(Nk/32)] or None): use
                these codes (and, for MXFP4, block exponents of blocks with a
                live key) instead of rounding; every other step is unchanged
    return_pre  also return the value each code rounds, [nq, Nk] (2**y for
                the exact encoders, the position 2**M (y + b) for the cast,
                -inf where masked), and the block maxima xmax of t - m',
                [nq, ceil(Nk/32)] (-inf for blocks with no live key)
    return_tiles  append a dict of the scales the accumulation ran at:
                "m_tile" [nq, ceil(Nk/128)] the running max m' each tile's
                probabilities are relative to (-inf for a tile with no live
                key), and the final "m" and "l" [nq]
    """
    if encoder not in ("exact", "loglin"):
        raise ValueError(encoder)
    q_raw = np.asarray(q_raw, np.float64)
    k_raw = np.asarray(k_raw, np.float64)
    v_hat = np.asarray(v_hat, np.float64)
    nq, Nk = q_raw.shape[0], k_raw.shape[0]
    if q_index is None:
        q_index = np.arange(nq)
    q_index = np.asarray(q_index)
    c = float(sigma) * LOG2E * float(np.float32(gq)) * float(np.float32(gk))
    t_all = c * (q_raw @ k_raw.T)
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    o = np.zeros((nq, v_hat.shape[1]))
    nblk = (Nk + PBLOCK - 1) // PBLOCK
    return_p = return_p or return_pre
    p_codes = np.zeros((nq, Nk), np.uint8) if return_p else None
    p_e8m0 = np.zeros((nq, nblk), np.uint8) if (return_p and p_format == "mxfp4") else None
    pre_all = np.full((nq, Nk), -np.inf) if return_pre else None
    xmax_all = np.full((nq, nblk), -np.inf) if return_pre else None
    m_tile = np.full((nq, (Nk + TILE - 1) // TILE), -np.inf) if return_tiles else None
    for t0 in range(0, Nk, TILE):
        t1 = min(t0 + TILE, Nk)
        keys = np.arange(t0, t1)
        live = np.ones((nq, t1 - t0), bool)
        if causal:
            live &= keys[None, :] <= q_index[:, None]
        any_live = live.any(axis=1)
        if not any_live.any():
            continue
        t = np.where(live, t_all[:, t0:t1], -np.inf)
        m_new = np.where(any_live, np.maximum(m, t.max(axis=1)), m)
        alpha = np.where(any_live, np.where(np.isneginf(m), 0.0, np.exp2(m - m_new)), 1.0)
        ms = np.where(any_live, m_new, 0.0)
        x = t - ms[:, None]                       # -inf where masked
        p_hat = np.zeros_like(x)
        for b0 in range(0, t1 - t0, PBLOCK):
            b1 = min(b0 + PBLOCK, t1 - t0)
            xb = x[:, b0:b1]
            lb = live[:, b0:b1]
            blk = (t0 + b0) // PBLOCK
            xmax = xb.max(axis=1)
            if return_pre:
                xmax_all[:, blk] = xmax
            if p_format == "mxfp4":
                has = lb.any(axis=1)
                e = np.where(has, np.maximum(np.floor(np.where(has, xmax, 0.0)) - 2, -127), -127)
                if p_given is not None:
                    e = np.where(has, p_given[1][:, blk].astype(np.int64) - 127, e)
                if encoder == "exact":
                    pre = np.exp2(xb - e[:, None])
                    codes = e2m1_encode(pre)
                else:
                    pre = loglin_position(xb - e[:, None], "e2m1")
                    codes = loglin_encode(xb - e[:, None], "e2m1")
                if p_given is not None:
                    codes = p_given[0][:, t0 + b0:t0 + b1]
                codes = np.where(lb, codes, 0).astype(np.uint8)
                p_hat[:, b0:b1] = e2m1_decode(codes) * np.exp2(e)[:, None]
                if return_p:
                    p_e8m0[:, blk] = (e + 127).astype(np.uint8)
            elif p_format == "fp8":
                if encoder == "exact":
                    pre = np.exp2(xb)
                    codes = e4m3_encode(pre)
                else:
                    pre = loglin_position(xb, "e4m3")
                    codes = loglin_encode(xb, "e4m3")
                if p_given is not None:
                    codes = p_given[0][:, t0 + b0:t0 + b1]
                codes = np.where(lb, codes, 0).astype(np.uint8)
                p_hat[:, b0:b1] = e4m3_decode(codes)
            else:
                raise ValueError(p_format)
            if return_p:
                p_codes[:, t0 + b0:t0 + b1] = codes
            if return_pre:
                pre_all[:, t0 + b0:t0 + b1] = np.where(lb, pre, -np.inf)
        l = alpha * l + p_hat.sum(axis=1)
        o = alpha[:, None] * o + p_hat @ v_hat[t0:t1]
        m = m_new
        if return_tiles:
            m_tile[:, t0 // TILE] = np.where(any_live, m_new, -np.inf)
    with np.errstate(divide="ignore", invalid="ignore"):
        O = np.where(l[:, None] > 0, o / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse = np.where(l > 0, LN2 * (m + np.log2(np.where(l > 0, l, 1.0))), -np.inf)
    tiles = ({"m_tile": m_tile, "m": m, "l": l},) if return_tiles else ()
    if return_pre:
        return (O, lse, p_codes, p_e8m0, pre_all, xmax_all) + tiles
    if return_p:
        return (O, lse, p_codes, p_e8m0) + tiles
    return (O, lse) + tiles


def attn_exact_head(q, k, v, sigma, causal=False, q_index=None):
    """Textbook softmax attention in float64 for one head:
    O = softmax(sigma * q k^T) v, LSE = log sum exp(sigma * q k^T)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    nq, Nk = q.shape[0], k.shape[0]
    if q_index is None:
        q_index = np.arange(nq)
    s = float(sigma) * (q @ k.T)
    if causal:
        s = np.where(np.arange(Nk)[None, :] <= np.asarray(q_index)[:, None], s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    w = np.exp(s - mx)
    den = w.sum(axis=1, keepdims=True)
    return (w @ v) / den, (mx + np.log(den))[:, 0]
