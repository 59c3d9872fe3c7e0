"""Pins of the oracle's attention backward (oracle.backward).

* Without quantization the oracle's dQ, dK, dV must equal automatic
  differentiation of textbook softmax attention (float64, CPU): this fixes
  the calculus (the D term, sigma, the transposes, the causal mask).
* The MX E4M3 and E5M2 quantizers are pinned by closed forms.
* A hand-derived case whose probabilities span 2^20 between two queries
  fixes where the MX blocks run: along queries for P~ and dS~K (dV, dK),
  along keys for dS~Q (dQ).
"""

import math

import numpy as np
import pytest
import torch

from oracle import backward as B
from oracle import formats as F

LN2 = math.log(2.0)


def _autograd(q_hat, k_hat, v, do, sigma, causal):
    q = torch.tensor(q_hat, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(k_hat, dtype=torch.float64, requires_grad=True)
    vv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    s = sigma * (q @ k.T)
    if causal:
        n, m = s.shape
        s = s.masked_fill(torch.arange(m)[None, :] > torch.arange(n)[:, None], float("-inf"))
    lse = torch.logsumexp(s, dim=1)
    o = torch.softmax(s, dim=1) @ vv
    (o * torch.tensor(do, dtype=torch.float64)).sum().backward()
    return o.detach().numpy(), lse.detach().numpy(), q.grad.numpy(), k.grad.numpy(), vv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 8), (37, 16), (130, 64)])
def test_unquantized_equals_autograd(causal, n, d):
    rng = np.random.default_rng(n + d + causal)
    q_raw = rng.standard_normal((n, d))
    k_raw = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    do = rng.standard_normal((n, d))
    gq, gk = np.float32(0.75), np.float32(1.25)
    sigma = 1 / math.sqrt(d)
    o, lse, dq, dk, dv = _autograd(q_raw * float(gq), k_raw * float(gk), v, do, sigma, causal)
    rq, rk, rv = B.attn_bwd_head(q_raw, k_raw, gq, gk, v, o, do, lse, sigma, causal, quantize=False)
    for got, want in ((rq, dq), (rk, dk), (rv, dv)):
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_row_and_column_subsets():
    rng = np.random.default_rng(3)
    n, d = 90, 16
    args = [rng.standard_normal((n, d)) for _ in range(5)]
    lse = rng.standard_normal(n) + 3.0
    full = B.attn_bwd_head(args[0], args[1], 1.0, 1.0, args[2], args[3], args[4], lse, 0.3, True)
    qr, kr = np.array([0, 5, 64, 89]), np.array([1, 31, 32, 88])
    part = B.attn_bwd_head(args[0], args[1], 1.0, 1.0, args[2], args[3], args[4], lse, 0.3, True,
                           q_rows=qr, k_rows=kr)
    np.testing.assert_array_equal(part[0], full[0][qr])
    np.testing.assert_array_equal(part[1], full[1][kr])
    np.testing.assert_array_equal(part[2], full[2][kr])


def test_mx_e4m3_closed_forms():
    # block max 1 -> e = 0 - 8; 1 * 2^8 = 256 and 0.5 * 2^8 = 128 are exact
    x = np.zeros(40)
    x[0], x[1], x[2] = 1.0, 0.5, -0.3
    deq, codes, e = B.mx_e4m3(x, axis=0)
    assert e.tolist() == [-8, -127]                  # second block (8 zeros) is empty
    assert deq[0] == 1.0 and deq[1] == 0.5
    assert deq[2] == F.e4m3_decode(F.e4m3_encode(-0.3 * 256)) / 256
    # the MX rule saturates a block whose max significand is >= 1.75 + 1/16:
    # 1.9 -> 1.9 * 2^8 = 486.4 -> 448 -> 1.75
    y = np.array([1.9, 1.0])
    assert B.mx_e4m3(y, axis=0)[0].tolist() == [1.75, 1.0]
    # scaled by 2^8, values under half the smallest subnormal (2^-10) flush to 0:
    # 2^-19 -> 2^-11 -> 0; 3 * 2^-17 -> 3 * 2^-9 is subnormal code 3, exact
    z = np.array([1.0, 2.0 ** -19, 3 * 2.0 ** -17])
    assert B.mx_e4m3(z, axis=0)[0].tolist() == [1.0, 0.0, 3 * 2.0 ** -17]


def test_mx_e4m3_axis():
    x = np.array([[1.0, 2.0 ** -20], [2.0 ** -20, 2.0 ** -20]])
    along0 = B.mx_e4m3(x, axis=0)[0]   # column 1 block: max 2^-20 keeps both
    along1 = B.mx_e4m3(x, axis=1)[0]   # row 0 block: max 1 flushes 2^-20
    assert along0.tolist() == [[1.0, 2.0 ** -20], [0.0, 2.0 ** -20]]
    assert along1.tolist() == [[1.0, 0.0], [2.0 ** -20, 2.0 ** -20]]


def test_e5m2_do_quantizer():
    # amax = 57344 -> enc = 1: codes are the E5M2 codes of the values themselves
    x = np.array([[57344.0, 1.0, -0.375, 3.0 * 2 ** -16, 0.1]], np.float32)
    codes, s = B.quant_do_e5m2(x)
    assert s == 1.0
    np.testing.assert_array_equal(codes, F.e5m2_encode(x))
    deq = B.dequant_do_e5m2(codes, s)
    assert deq[0, :4].tolist() == [57344.0, 1.0, -0.375, 3.0 * 2 ** -16]
    # zero tensor: scale 1, codes 0
    codes, s = B.quant_do_e5m2(np.zeros((2, 3), np.float32))
    assert s == 1.0 and not codes.any()
    # amax 7 -> enc = fl(57344 / 7): the largest element maps to 57344 up to rounding
    codes, s = B.quant_do_e5m2(np.array([7.0, -7.0], np.float32))
    assert codes.tolist() == [0x7B, 0xFB]


def _span_case():
    """Two queries, four keys, D = 2, sigma = ln 2, g = 1: t_ij = t_j + u_i.
    LSE chosen so that P_0j = 2^-j and P_1j = 2^(-20-j).  V = 0 and O, dO
    chosen so that D_i = -1: dS = P."""
    t = np.array([0.0, -1.0, -2.0, -3.0])
    u = np.array([3.0, -2.0])
    a = np.array([0.0, 20.0])
    q_raw = np.stack([np.ones(2), u], axis=1)
    k_raw = np.stack([t, np.ones(4)], axis=1)
    lse = (u + a) * LN2
    v = np.zeros((4, 2))
    do = np.array([[1.0, 0.0], [0.0, 1.0]])
    o = np.array([[-1.0, 0.0], [0.0, -1.0]])
    return q_raw, k_raw, v, o, do, lse, t, u


def test_hand_derived_block_axes():
    q_raw, k_raw, v, o, do, lse, t, u = _span_case()
    dq, dk, dv = B.attn_bwd_head(q_raw, k_raw, 1.0, 1.0, v, o, do, lse, LN2)
    p0 = np.exp2(-np.arange(4.0))
    # dV: P~ in blocks along queries; per key the block {P_0j, P_1j} has max P_0j,
    # and P_1j = 2^-20 P_0j falls under E4M3's smallest subnormal: dV_j = [P_0j, 0]
    np.testing.assert_allclose(dv, np.stack([p0, np.zeros(4)], axis=1), rtol=1e-12, atol=0)
    # dK: dS~K = P~: dK_j = ln2 P_0j (1, u_0)
    np.testing.assert_allclose(dk, LN2 * p0[:, None] * np.array([1.0, u[0]])[None, :], rtol=1e-12, atol=0)
    # dQ: dS~Q in blocks along keys keeps row 1 exactly (powers of two):
    # dQ_i = ln2 sum_j P_ij (t_j, 1)
    k_hat = np.stack([t, np.ones(4)], axis=1)
    want = LN2 * np.stack([p0 @ k_hat, 2.0 ** -20 * (p0 @ k_hat)])
    np.testing.assert_allclose(dq, want, rtol=1e-12, atol=0)
    # unquantized, dV keeps the second query
    _, _, dv_exact = B.attn_bwd_head(q_raw, k_raw, 1.0, 1.0, v, o, do, lse, LN2, quantize=False)
    np.testing.assert_allclose(dv_exact[:, 1], 2.0 ** -20 * p0, rtol=1e-12)


def test_quantized_close_to_unquantized():
    # not parity: a sanity bound on the quantization error of realistic inputs
    rng = np.random.default_rng(11)
    n, d = 200, 64
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    o, lse, *_ = _autograd(q, k, v, do, 0.125, True)
    codes, s = B.quant_do_e5m2(do.astype(np.float32))
    do_hat = B.dequant_do_e5m2(codes, s)
    got = B.attn_bwd_head(q, k, 1.0, 1.0, v, o, do_hat, lse, 0.125, True)
    ref = B.attn_bwd_head(q, k, 1.0, 1.0, v, o, do, lse, 0.125, True, quantize=False)
    for g, r in zip(got, ref):
        assert np.linalg.norm(g - r) / np.linalg.norm(r) < 0.2
