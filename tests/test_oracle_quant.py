"""Pins of the oracle's quantizers: hand-derived blocks, exact round trips on
representable tensors, power-of-two equivariance and the degenerate cases."""

import numpy as np

from oracle import quant as Q
from oracle import formats as F


def test_nvfp4_hand_derived_two_blocks():
    # Row of 32 values (two 16-element blocks), all exact in bf16.
    b0 = [6.0, -3.0, 1.25, 0.6875, 2.625, -5.125, 0.203125, 4.375,
          0.0, -0.2578125, 1.75, 3.5, 0.75, -1.0, 5.0, 2.5]
    b1 = [0.5, 0.25, -0.125, 0.0625, 0.1875, -0.3125, 0.375, 0.4375,
          0.03125, 0.09375, -0.5, 0.15625, 0.2734375, 0.0, 0.46875, -0.0390625]
    codes, scales, g = Q.quant_nvfp4(np.array([b0 + b1], np.float32))
    # amax_t = 6 -> S_enc = 2688/6 = 448 exactly; g = fl32(1/448).
    assert g == np.float32(1.0) / np.float32(448.0)
    # Block 0: amax_b = 6 -> s = E4M3(6/6 * 448) = 448 = 0x7E; enc = 1, so the
    # codes are E2M1(x): 6->7, -3->13, 1.25 (tie 1|1.5)->2, 0.6875->1,
    # 2.625->5, -5.125->15, 0.203125->0, 4.375->6, 0->0, -0.2578125->9,
    # 1.75 (tie)->4, 3.5 (tie)->6, 0.75 (tie)->2, -1->10, 5 (tie)->6, 2.5 (tie)->4.
    # Block 1: amax_b = 0.5 -> fl(0.5/6) * 448 = 37.333336 -> E4M3 36 (2**5 * 1.125,
    # code 0x61); enc = fl(448/36) = 12.444445; x*enc then E2M1:
    # 6.22->7, 3.11->5, -1.56->11, 0.78->2, 2.33->4, -3.89->14, 4.67->6,
    # 5.44->7, 0.39->1, 1.17->2, -6.22->15, 1.94->4, 3.40->5, 0->0, 5.83->7, -0.49->9.
    assert scales.tolist() == [[0x7E, 0x61]]
    assert codes.tolist() == [[0xD7, 0x12, 0xF5, 0x60, 0x90, 0x64, 0xA2, 0x46,
                               0x57, 0x2B, 0xE4, 0x76, 0x21, 0x4F, 0x05, 0x97]]


def _representable_nvfp4(rng, rows, D, k):
    """A tensor that NVFP4 must reproduce exactly: amax_t = 2688 * 2**k makes
    S_enc = 2**-k and g = 2**k; each block holds one E2M1 6 (so its amax is
    6 * s * 2**k and its scale is s) and other E2M1 multiples of s * 2**k."""
    e4m3_vals = F.e4m3_decode(np.arange(1, 0x7F))     # positive finite, non-zero
    e4m3_vals = e4m3_vals[(e4m3_vals >= 2.0 ** -6)]   # keep block scales normal
    nb = D // 16
    s = rng.choice(e4m3_vals, size=(rows, nb))
    s[0, 0] = 448.0
    c = rng.integers(0, 16, size=(rows, nb, 16)).astype(np.uint8)
    c[..., 0] = 7                                        # the block max: +6
    x = F.e2m1_decode(c) * s[..., None] * 2.0 ** k
    return x.reshape(rows, D).astype(np.float32), c.reshape(rows, D), s


def test_nvfp4_exact_round_trip():
    rng = np.random.default_rng(1)
    for k in (-8, 0, 5):
        x, c, s = _representable_nvfp4(rng, 64, 128, k)
        codes, scales, g = Q.quant_nvfp4(x)
        assert g == np.float32(2.0 ** k)
        np.testing.assert_array_equal(F.e4m3_decode(scales), s)
        got = F.unpack_nibbles(codes)
        # a stored +0/-0 may differ only in the zero's sign, which decodes equal
        np.testing.assert_array_equal(F.e2m1_decode(got), F.e2m1_decode(c))
        np.testing.assert_array_equal(Q.dequant_nvfp4(codes, scales, g), x.astype(np.float64))


def test_nvfp4_power_of_two_equivariance():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    c1, s1, g1 = Q.quant_nvfp4(x)
    c2, s2, g2 = Q.quant_nvfp4(x * np.float32(2))
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)
    assert g2 == 2 * g1


def test_nvfp4_error_bound():
    # |x*enc - E2M1(code)| is at most half the E2M1 spacing at that magnitude,
    # plus whatever lies beyond the saturation point 6.
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((128, 128)) * np.exp2(rng.uniform(-6, 6, (128, 1)))).astype(np.float32)
    codes, scales, g = Q.quant_nvfp4(x)
    s = F.e4m3_decode(scales)
    amax_t = np.abs(x).max()
    s_enc = np.float32(np.float32(2688) / np.float32(amax_t))
    enc = np.repeat((s_enc / s.astype(np.float32)).astype(np.float32), 16, axis=1)
    y = np.abs(x.astype(np.float64) * enc)
    dq = np.abs(F.e2m1_decode(F.unpack_nibbles(codes)))
    spacing = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    assert np.all(np.abs(y - dq) <= spacing / 2 + np.maximum(0, y - 6) + 1e-6)


def test_nvfp4_zero_and_underflowing_block():
    codes, scales, g = Q.quant_nvfp4(np.zeros((4, 32), np.float32))
    assert g == 1.0 and not codes.any() and not scales.any()
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1000.0
    x[0, 16:] = -1e-6          # amax_b/6 * S_enc = 4.5e-7, below E4M3's 2**-10
    codes, scales, g = Q.quant_nvfp4(x)
    assert scales[0, 1] == 0
    assert not F.unpack_nibbles(codes)[0, 16:].any()


def test_mx_exponent_rule():
    # OCP MX for E2M1: e = floor(log2(amax)) - 2
    assert Q.mx_block_exponent([1.0, 0.99, 7.0, 6.0, 2.0 ** -130, 0.0]).tolist() == \
        [-2, -3, 0, 0, -127, -127]


def test_mxfp4_v_round_trip_and_equivariance():
    rng = np.random.default_rng(4)
    Nk, H, D = 70, 2, 8          # a short last block of 6 keys
    nblk = 3
    k = rng.integers(-20, 20, size=(nblk, H, D))
    c = rng.integers(0, 16, size=(nblk * 32, H, D)).astype(np.uint8)
    c[0::32] = 7                  # first key of each block holds +6
    v = (F.e2m1_decode(c) * np.repeat(np.exp2(k), 32, axis=0))[:Nk].astype(np.float32)
    codes, e8 = Q.quant_v_mxfp4(v)
    np.testing.assert_array_equal(e8.astype(int) - 127, k)
    np.testing.assert_array_equal(Q.dequant_v_mxfp4(codes, e8), v.astype(np.float64))
    codes2, e82 = Q.quant_v_mxfp4(v * np.float32(2))
    np.testing.assert_array_equal(codes, codes2)
    np.testing.assert_array_equal(e82.astype(int), e8.astype(int) + 1)


def test_mxfp4_v_zero_block_and_saturation():
    v = np.zeros((40, 1, 2), np.float32)
    v[:32, 0, 1] = 1.75           # amax 1.75 -> e = -2 -> 7.0 saturates to 6
    codes, e8 = Q.quant_v_mxfp4(v)
    assert e8[:, 0, 0].tolist() == [0, 0]                # all-zero blocks: e = -127
    assert e8[0, 0, 1] == 125 and codes[0, 0, 1] == 7
    assert not codes[:, 0, 0].any()


def test_fp8_v_round_trip():
    rng = np.random.default_rng(5)
    vals = F.e4m3_decode(rng.integers(0, 0x7E, size=(50, 3, 16)))
    vals[0, 0, 0] = 448.0
    for k in (-3, 0, 4):
        v = (vals * 2.0 ** k).astype(np.float32)
        codes, s_v = Q.quant_v_fp8(v)
        assert s_v == np.float32(2.0 ** k)
        np.testing.assert_array_equal(Q.dequant_v_fp8(codes, s_v), v.astype(np.float64))
    codes, s_v = Q.quant_v_fp8(np.zeros((3, 1, 4), np.float32))
    assert s_v == 1.0 and not codes.any()


# FP8 V with a non-power-of-two amax.  The rule: enc = fl(448 / amax),
# stored scale s_v = fl(1 / enc), code = E4M3(fl(v * enc)) -- the NVFP4 tensor
# scale's pattern.  Hand-derived with exact rational arithmetic and
# round-to-nearest-even to float32 / E4M3, for amax = 1.53125 = 49/32:
#   448 / amax = 292.571428...; its float32 rounding enc = 0x43924925 (292.57144165).
#   1 / enc = 0.00341796851...; float32 s_v = 0x3B5FFFFF, one ulp below
#   amax / 448 = 7/2048 = 0x3B600000 (which the rule s_v = fl(amax / 448)
#   would store).
#   v = 91 * 2^-21: v * enc = 0.0126953134 > 13 * 2^-10, the midpoint of the
#   E4M3 subnormals 6 * 2^-9 and 7 * 2^-9, so the code is 7; dividing by
#   7/2048 instead would land exactly on the midpoint and tie to the even 6.
#   1.0 -> 292.571 -> nearest 288 (1.125 * 2^8, code 0x79); -0.5 -> 146.29 ->
#   144 (0xF1); 0.75 -> 219.43 -> 224 (1.75 * 2^7, 0x76); 2^-10 -> 0.2857 ->
#   0.28125 (1.125 * 2^-2, 0x29); +-amax -> 448.00003 saturates to 448 (0x7E).
FP8V_AMAX_PIN = {
    "values": [49 / 32, -49 / 32, 1.0, -0.5, 91 * 2.0 ** -21, -91 * 2.0 ** -21, 0.0, 0.75, 2.0 ** -10],
    "codes": [0x7E, 0xFE, 0x79, 0xF1, 0x07, 0x87, 0x00, 0x76, 0x29],
    "s_v_bits": 0x3B5FFFFF,
}


def test_fp8_v_scale_non_power_of_two_amax():
    v = np.array(FP8V_AMAX_PIN["values"], np.float32).reshape(3, 1, 3)
    codes, s_v = Q.quant_v_fp8(v)
    assert np.float32(s_v).view(np.uint32) == FP8V_AMAX_PIN["s_v_bits"]
    assert codes.reshape(-1).tolist() == FP8V_AMAX_PIN["codes"]
    # the stored scale is not amax / 448 rounded once (that would be 0x3B600000)
    assert np.float32(np.float32(49 / 32) / np.float32(448)).view(np.uint32) == 0x3B600000
