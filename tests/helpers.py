"""Shared test plumbing: run the oracle and the HIP path on the same seeded
inputs and compare.  The oracle never sees anything the HIP path produced."""

import math

import numpy as np
import torch

from oracle import attention as OA
from oracle import formats as OF
from oracle import quant as OQ

# Tolerances of the parity bar (float results); codes and scales are bit-exact.
P_MISMATCH_MAX = 1e-4        # fraction of live probability codes
O_REL_L2_MAX = 1e-3
O_MAX_ABS = 5e-3
LSE_REL_MAX = 1e-4           # |dLSE| <= 1e-4 * max(1, |LSE|)


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
                q_index=None, return_p=False):
    """Oracle forward for a set of query rows of one head, given the bf16
    inputs (as float32 numpy) and the whole-tensor amax values."""
    qc, qs, gq = OQ.quant_nvfp4(q_rows, amax=amax_q)
    kc, ks, gk = OQ.quant_nvfp4(k_rows, amax=amax_k)
    vh = oracle_v_head(v_rows, v_format, amax_v)
    return OA.attn_lowp_head(OQ.dequant_nvfp4_raw(qc, qs), OQ.dequant_nvfp4_raw(kc, ks), gq, gk, vh, sigma,
                             p_format, causal, q_index=q_index, return_p=return_p)


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
