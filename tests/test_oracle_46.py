"""Pins of the oracle's Four Over Six NVFP4 quantizer (oracle.quant.quant_nvfp4_46).

Only the abstract is on the pages.  The pins are hand-derived blocks (one
that the max-4 scale represents exactly where the max-6 scale does not, one
where max-6 is better), the exact float64 squared error of the chosen block
against both single-candidate quantizations, degenerate inputs, and the
format itself (dequantize(quantize(x)) = x on representable values).
"""

import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q


def _deq(codes, scales, g):
    return Q.dequant_nvfp4(codes, scales, g)


def test_hand_derived_block_where_four_is_exact():
    # amax_t = 7 -> S_enc = 1792/7 = 256, g = 1/256 (exact).
    # M = 6: s = E4M3(7/6 * 256 = 298.67) = 288, enc = 256/288: 7 -> 6.22 -> 6,
    #   5.25 -> 4.67 -> 4: squared error (1792-1728)^2 + (1344-1152)^2 = 40960.
    # M = 4: s = E4M3(448) = 448, enc = 256/448: 7 -> 4, 5.25 -> 3 exactly, error 0 -> M = 4.
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1] = 7.0, 5.25
    c, s, g, four = Q.quant_nvfp4_46(x, return_choice=True)
    assert four.tolist() == [[True]]
    assert s.tolist() == [[0x7E]] and F.e4m3_decode(0x7E) == 448.0
    assert F.unpack_nibbles(c)[0, :2].tolist() == [6, 5]          # E2M1 4.0 and 3.0
    assert g == np.float32(1.0 / 256.0)
    np.testing.assert_array_equal(_deq(c, s, g), x)
    # the standard recipe (max 6, S_enc = 2688/amax) maps 5.25 to 4.67 here
    c6, s6, g6 = Q.quant_nvfp4(x)
    assert abs(_deq(c6, s6, g6)[0, 1] - 5.25) > 0.5


def test_hand_derived_block_where_six_wins():
    # amax_t = 6 -> S_enc = 298.67.  M = 6: s = 288: 6 -> 1728 (d 64), 1 -> 288 (d 10.7):
    # error ~ 4210.  M = 4: s = 448: 6 -> 4 (d 0), 1 -> 0.667 -> 0.5 (d 74.7): error ~ 5575.
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1] = 6.0, 1.0
    c, s, g, four = Q.quant_nvfp4_46(x, return_choice=True)
    assert four.tolist() == [[False]]
    assert F.e4m3_decode(s[0, 0]) == 288.0
    assert F.unpack_nibbles(c)[0, :2].tolist() == [7, 2]          # E2M1 6.0 and 1.0


def _block_err(x, codes, scales, g):
    """Exact squared error per block, float64."""
    d = _deq(codes, scales, g) - x.astype(np.float64)
    return (d.reshape(d.shape[0], -1, 16) ** 2).sum(-1)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_chosen_block_is_never_worse_than_either_candidate(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[:, rng.integers(0, 128, 4)] *= 8.0
    amax = np.abs(x).max()
    both = Q.quant_nvfp4_46(x, amax=amax, return_choice=True)
    e = _block_err(x, *both[:3])
    e6 = _block_err(x, *Q.quant_nvfp4_46(x, amax=amax, candidates=(6.0,)))
    e4 = _block_err(x, *Q.quant_nvfp4_46(x, amax=amax, candidates=(4.0,)))
    slack = 1e-5 * np.maximum(e6, e4) + 1e-30
    assert np.all(e <= np.minimum(e6, e4) + slack)
    # both candidates are taken somewhere on Gaussian data
    assert 0.05 < both[3].mean() < 0.95
    # and the total error is below that of the max-6 recipe alone
    assert e.sum() < e6.sum()


def test_zero_tensor_and_zero_block():
    c, s, g = Q.quant_nvfp4_46(np.zeros((2, 32), np.float32))
    assert not c.any() and not s.any() and g == 1.0
    x = np.zeros((1, 32), np.float32)
    x[0, 20] = 7.0                    # S_enc = 256: the max-4 scale 448 holds 7 exactly
    c, s, g = Q.quant_nvfp4_46(x)
    assert s[0, 0] == 0 and not F.unpack_nibbles(c)[0, :16].any()
    np.testing.assert_array_equal(_deq(c, s, g), x)


def test_representable_values_round_trip():
    # values E2M1 * 448 / 256 (amax 7, S_enc 256, g exact): the max-4 grid of every block
    rng = np.random.default_rng(5)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4], np.float32) * np.float32(1.75)
    x = rng.choice(mags, (8, 64)) * rng.choice([-1, 1], (8, 64)).astype(np.float32)
    x[:, ::16] = 7.0
    c, s, g = Q.quant_nvfp4_46(x)
    np.testing.assert_array_equal(_deq(c, s, g), x)


def test_tie_keeps_the_standard_scale():
    # amax_t = 7 (another block) -> S_enc = 256.  Block [6]: M = 6 gives s = 256, enc 1,
    # code 6.0; M = 4 gives s = 384, 6 -> 4.0: both exact, equal errors -> M = 6 (E4M3 256 = 0x78).
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 7.0
    x[0, 16] = 6.0
    c, s, g, four = Q.quant_nvfp4_46(x, return_choice=True)
    assert four.tolist() == [[True, False]]
    assert s[0, 1] == 0x78 and F.e4m3_decode(0x78) == 256.0
    np.testing.assert_array_equal(_deq(c, s, g), x)
