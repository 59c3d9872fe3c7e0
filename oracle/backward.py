"""Backward of the low-precision attention (causal training path) in the oracle.
TEST INFRASTRUCTURE ONLY.

Follows "Hardware-Aware FP4 FlashAttention-4" (summary page, "What the paper
found", and the abstract on the arXiv listing 2609.04105v1): for causal
training the forward keeps its quantized Q/K payloads, their scales and the
LSE; the backward rebuilds the probabilities from them and runs its products
on FP8 gradient operands, the output gradient dO in E5M2; training keeps FP8
P and V.  The pages give no formulas.  Readings taken, each the plain
FlashAttention-style backward restated with those operands:

1. Inputs per (batch, head): the forward's exact NVFP4 values Q_raw, K_raw
   (E2M1 * E4M3, tensor scales g_q, g_k), its dequantized FP8 V, its output O
   as stored, its LSE, and dO.
2. dO is quantized to E5M2 with one FP32 scale per tensor, as FP8 V is to
   E4M3: S = fl(57344 / amax), code = E5M2(fl(dO * S)), s = fl(1 / S).
3. P_ij = 2^(t_ij - LSE_i * log2 e) with t = c * Q_raw . K_raw and
   c = sigma * log2 e * g_q * g_k as in the forward; masked keys give 0.
4. D_i = sum_d dO^_id O_id, dP = dO^ V^T, dS = P * (dP - D).
5. FP8 operands take E4M3 codes with one E8M0 exponent per 32 consecutive
   elements along the contraction axis of the product they enter (the OCP MX
   rule: e = max(floor(log2 amax) - 8, -127), code = E4M3(x * 2^-e), blocks
   aligned to index 0 of the sequence):
     P~   for dV = P~^T dO^      : blocks of 32 queries, per key;
     dS~K for dK = sigma dS~K^T Q^ : blocks of 32 queries, per key;
     dS~Q for dQ = sigma dS~Q K^   : blocks of 32 keys, per query.
   Q^ = Q_raw g_q and K^ = K_raw g_k are the exact NVFP4 values.
With ``quantize=False`` the E5M2 and MX steps are skipped (dO^ = dO, P~ = P,
dS~ = dS): the textbook softmax-attention backward, which the tests compare
with automatic differentiation.

All arithmetic is float64.
"""

import math

import numpy as np

from .formats import e4m3_encode, e4m3_decode, e5m2_encode, e5m2_decode

F32 = np.float32
LOG2E = 1.0 / math.log(2.0)
MX_BLOCK = 32
E4M3_EMAX = 8          # largest E4M3 value 1.75 * 2^8


def quant_do_e5m2(do, amax=None):
    """E5M2 dO with one FP32 scale per tensor (reading 2).  Returns (codes
    uint8 like do, s float32); the dequantized value is E5M2(code) * s."""
    do = np.asarray(do, dtype=F32)
    if amax is None:
        amax = np.max(np.abs(do)) if do.size else 0.0
    amax = F32(amax)
    enc = F32(1.0) if amax == 0 else F32(F32(57344.0) / amax)
    if not np.isfinite(enc):
        enc = F32(np.finfo(np.float32).max)
    codes = e5m2_encode((do * enc).astype(F32))
    return codes, F32(F32(1.0) / enc)


def dequant_do_e5m2(codes, s):
    return e5m2_decode(codes) * np.float64(s)


def mx_e4m3(x, axis):
    """MX E4M3 quantization of float64 ``x`` in blocks of 32 along ``axis``
    (reading 5).  Returns (dequantized float64, codes uint8, exponents int64
    with the blocked axis shortened to ceil(n / 32))."""
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    nb = (n + MX_BLOCK - 1) // MX_BLOCK
    pad = nb * MX_BLOCK - n
    xp = np.concatenate([xm, np.zeros(xm.shape[:-1] + (pad,))], axis=-1) if pad else xm
    xb = xp.reshape(xm.shape[:-1] + (nb, MX_BLOCK))
    amax = np.abs(xb).max(axis=-1)
    with np.errstate(divide="ignore"):
        fl = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    e = np.where(amax > 0, np.maximum(fl - E4M3_EMAX, -127), -127).astype(np.int64)
    codes = e4m3_encode(xb * np.exp2(-e)[..., None])
    deq = e4m3_decode(codes) * np.exp2(e)[..., None]
    codes = codes.reshape(xp.shape)[..., :n]
    deq = deq.reshape(xp.shape)[..., :n]
    return np.moveaxis(deq, -1, axis), np.moveaxis(codes, -1, axis), np.moveaxis(e, -1, axis)


def _given_values(codes, exps, axis):
    """E4M3 codes times 2^e with the E8M0 bytes ``exps`` (e + 127) repeated
    over the 32-element blocks of ``axis``."""
    e = np.repeat(np.asarray(exps, np.int64) - 127, MX_BLOCK, axis=axis)
    e = e[:, :codes.shape[1]] if axis == 1 else e[:codes.shape[0], :]
    return e4m3_decode(codes) * np.exp2(e)


def attn_bwd_head(q_raw, k_raw, gq, gk, v_hat, o, do_hat, lse, sigma, causal=False,
                  q_rows=None, k_rows=None, quantize=True, given=None, return_pre=False):
    """Backward of one (batch, head) for a sequence of Nq queries and Nk keys.

    q_raw [Nq, D], k_raw [Nk, D]: exact NVFP4 values without tensor scales;
    v_hat [Nk, D]: dequantized V; o [Nq, D]: the forward output; do_hat
    [Nq, D]: the (dequantized E5M2) output gradient; lse [Nq]: natural-log LSE.
    q_rows / k_rows select the query rows of dQ and the key rows of dK, dV
    (default all); each needs every key / query, which the function computes.
    Returns (dQ [len(q_rows), D], dK [len(k_rows), D], dV [len(k_rows), D]).

    Hooks for checking an implementation whose float32 arithmetic may round a
    value lying on an E4M3 boundary the other way:
    given       dict with any of "ds_q" (codes [len(q_rows), Nk], E8M0 bytes
                [len(q_rows), ceil(Nk/32)]), "p_t" and "ds_k" (codes [Nq,
                len(k_rows)], E8M0 bytes [ceil(Nq/32), len(k_rows)]): use
                these instead of rounding; every other step is unchanged
    return_pre  also return a dict of intermediates: for "q" (the dQ rows)
                and "k" (the dK/dV columns) the exact P, dS, the codes and
                exponents, and the magnitude sums |Q_raw|.|K_raw|, |dO^|.|V^|
                and |dO^|.|O| (for error bounds of float32 sums)
    """
    q_raw = np.asarray(q_raw, np.float64)
    k_raw = np.asarray(k_raw, np.float64)
    v_hat = np.asarray(v_hat, np.float64)
    o = np.asarray(o, np.float64)
    do_hat = np.asarray(do_hat, np.float64)
    lse = np.asarray(lse, np.float64)
    Nq, Nk = q_raw.shape[0], k_raw.shape[0]
    q_rows = np.arange(Nq) if q_rows is None else np.asarray(q_rows)
    k_rows = np.arange(Nk) if k_rows is None else np.asarray(k_rows)
    c = float(sigma) * LOG2E * float(np.float32(gq)) * float(np.float32(gk))
    q_hat = q_raw * float(np.float32(gq))
    k_hat = k_raw * float(np.float32(gk))
    L = lse * LOG2E
    D_ = (do_hat * o).sum(axis=1)                              # reading 4

    def probs(qi, kj):
        t = c * (q_raw[qi] @ k_raw[kj].T)
        p = np.exp2(t - L[qi][:, None])
        if causal:
            p = np.where(kj[None, :] <= qi[:, None], p, 0.0)
        return p

    given = given or {}
    pre = {}
    # dQ rows: all keys, MX blocks along keys (per query row)
    kall = np.arange(Nk)
    p = probs(q_rows, kall)
    ds = p * (do_hat[q_rows] @ v_hat.T - D_[q_rows][:, None])
    ds_q = ds
    if quantize:
        ds_q, cq, eq = mx_e4m3(ds, axis=1)
        if "ds_q" in given:
            ds_q = _given_values(*given["ds_q"], axis=1)
        if return_pre:
            pre["q"] = dict(p=p, ds=ds, codes=cq, exps=eq + 127, D=D_[q_rows], abs_D=np.abs(do_hat * o).sum(1)[q_rows],
                            abs_qk=c * (np.abs(q_raw[q_rows]) @ np.abs(k_raw).T),
                            abs_dpv=np.abs(do_hat[q_rows]) @ np.abs(v_hat).T, lse2=L[q_rows])
    dq = sigma * (ds_q @ k_hat)

    # dK, dV rows: all queries, MX blocks along queries (per key column)
    qall = np.arange(Nq)
    p = probs(qall, k_rows)
    ds = p * (do_hat @ v_hat[k_rows].T - D_[:, None])
    p_t, ds_k = p, ds
    if quantize:
        p_t, cp, ep = mx_e4m3(p, axis=0)
        ds_k, ck, ek = mx_e4m3(ds, axis=0)
        if "p_t" in given:
            p_t = _given_values(*given["p_t"], axis=0)
        if "ds_k" in given:
            ds_k = _given_values(*given["ds_k"], axis=0)
        if return_pre:
            pre["k"] = dict(p=p, ds=ds, codes_p=cp, exps_p=ep + 127, codes_ds=ck, exps_ds=ek + 127, D=D_,
                            abs_D=np.abs(do_hat * o).sum(1),
                            abs_qk=c * (np.abs(q_raw) @ np.abs(k_raw[k_rows]).T),
                            abs_dpv=np.abs(do_hat) @ np.abs(v_hat[k_rows]).T, lse2=L)
    dv = p_t.T @ do_hat
    dk = sigma * (ds_k.T @ q_hat)
    if return_pre:
        return dq, dk, dv, pre
    return dq, dk, dv
