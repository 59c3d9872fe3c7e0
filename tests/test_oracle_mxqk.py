"""Pins of the oracle's MXFP4 Q/K quantizer (the opt-in MX-native Q/K format:
E2M1 elements, one E8M0 exponent per 32 elements along D): a hand-derived
row, brute-force nearest-value search on small random blocks, exact round
trips on representable rows, power-of-two equivariance and the degenerate
blocks."""

import math

import numpy as np

from oracle import quant as Q
from oracle import formats as F

E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_mxfp4_hand_derived_two_blocks():
    b0 = [5.0, -2.6, 0.3, 0.25, 0.75, 1.25, -0.0, 4.9] + [0.0] * 24
    b1 = [0.1, 0.05, -0.02, 0.0078125] + [0.0] * 28
    codes, e8 = Q.quant_mxfp4(np.array([b0 + b1], np.float32))
    # Block 0: amax 5 -> floor(log2 5) = 2 -> e = 0 (byte 127); codes E2M1(x):
    # 5 (tie 4|6) -> 4 = code 6, -2.6 -> -3 = 13, 0.3 -> 0.5 = 1,
    # 0.25 (tie 0|0.5) -> 0, 0.75 (tie) -> 1.0 = 2, 1.25 (tie) -> 1.0 = 2,
    # -0 -> 8, 4.9 -> 4 = 6.
    # Block 1: amax 0.1 -> floor(log2 0.1) = -4 -> e = -6 (byte 121); x * 64:
    # 6.4 -> saturates at 6 = 7, 3.2 -> 3 = 5, -1.28 -> -1.5 = 11, 0.5 = 1.
    assert e8.tolist() == [[127, 121]]
    expect = [0xD6, 0x01, 0x22, 0x68] + [0] * 12 + [0x57, 0x1B] + [0] * 14
    assert codes.tolist() == [expect]


def _nearest_code(y):
    """Brute force: the E2M1 code of the grid value nearest to y (ties to the
    even code), saturating at 6; sign bit kept for negative y and -0."""
    a = abs(y)
    best, bestd = 0, None
    for c, v in enumerate(E2M1_GRID):
        d = abs(a - v)
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    if a > 6.0:
        best = 7
    neg = y < 0 or (y == 0 and math.copysign(1.0, y) < 0)
    return best | (8 if neg else 0)


def test_mxfp4_brute_force_small():
    rng = np.random.default_rng(11)
    rows, D = 6, 64
    x = (rng.standard_normal((rows, D)) * np.exp2(rng.integers(-12, 12, (rows, 1)))).astype(np.float32)
    x[2, 5] = -0.0
    x[3, 32:64] = 0.0
    codes, e8 = Q.quant_mxfp4(x)
    cu = F.unpack_nibbles(codes)
    for r in range(rows):
        for blk in range(D // 32):
            vals = [float(v) for v in x[r, 32 * blk:32 * blk + 32]]
            amax = max(abs(v) for v in vals)
            if amax == 0:
                e = -127
            else:
                m, k = math.frexp(amax)          # amax = m 2**k, m in [0.5, 1)
                e = max(-127, min(127, (k - 1) - 2))
            assert int(e8[r, blk]) == e + 127
            for j, v in enumerate(vals):
                assert int(cu[r, 32 * blk + j]) == _nearest_code(math.ldexp(v, -e)), (r, blk, j, v)


def test_mxfp4_representable_round_trip():
    rng = np.random.default_rng(5)
    rows, D = 16, 128
    nb = D // 32
    codes = rng.integers(0, 16, (rows, D)).astype(np.uint8)
    codes[codes == 8] = 0                      # no -0 (it would read back as +0 codes)
    e = rng.integers(-30, 30, (rows, nb))
    # element 0 of every block is +-6 or +-4, so the block max fixes e exactly
    lead = rng.choice([7, 6, 15, 14], size=(rows, nb)).astype(np.uint8)
    for blk in range(nb):
        codes[:, 32 * blk] = lead[:, blk]
    x = (F.e2m1_decode(codes) * np.repeat(np.ldexp(1.0, e), 32, axis=1)).astype(np.float32)
    got_c, got_e = Q.quant_mxfp4(x)
    assert np.array_equal(got_e, (e + 127).astype(np.uint8))
    assert np.array_equal(F.unpack_nibbles(got_c), codes)
    assert np.array_equal(Q.dequant_mxfp4(got_c, got_e), x.astype(np.float64))


def test_mxfp4_power_of_two_equivariance():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    c1, e1 = Q.quant_mxfp4(x)
    c2, e2 = Q.quant_mxfp4(x * np.float32(2.0))
    c3, e3 = Q.quant_mxfp4(x * np.float32(0.25))
    assert np.array_equal(c1, c2) and np.array_equal(c1, c3)
    assert np.array_equal(e2.astype(int), e1.astype(int) + 1)
    assert np.array_equal(e3.astype(int), e1.astype(int) - 2)


def test_mxfp4_degenerate_blocks():
    x = np.zeros((3, 64), np.float32)
    x[1, :32] = np.float32(2.0 ** -130)         # block max far below the E8M0 range
    x[2, 40] = np.float32(-7.0)                 # lone value: e = 0, saturates to -6
    codes, e8 = Q.quant_mxfp4(x)
    cu = F.unpack_nibbles(codes)
    assert e8[0].tolist() == [0, 0] and not cu[0].any()
    assert e8[1].tolist() == [0, 0] and not cu[1].any()   # 2**-130 * 2**127 = 0.125 -> 0
    assert e8[2].tolist() == [0, 127]
    assert cu[2, 40] == 15 and cu[2].sum() == 15
    assert Q.dequant_mxfp4(codes, e8)[2, 40] == -6.0


def _sylvester(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_hadamard32_is_the_sylvester_matrix():
    # small integers: every float32 sum is exact, so the butterfly must equal
    # the matrix product with the Sylvester Hadamard matrix built by Kronecker
    # products, block by block
    rng = np.random.default_rng(3)
    x = rng.integers(-50, 50, (5, 64)).astype(np.float32)
    H = _sylvester(32)
    want = np.concatenate([x[:, :32].astype(np.float64) @ H.T, x[:, 32:].astype(np.float64) @ H.T], axis=1)
    assert np.array_equal(Q.hadamard32(x).astype(np.float64), want)
    assert np.array_equal(H @ H.T, 32 * np.eye(32))


def test_hadamard32_orthogonality_and_dot_products():
    rng = np.random.default_rng(4)
    q = rng.integers(-20, 20, (3, 128)).astype(np.float32)
    k = rng.integers(-20, 20, (4, 128)).astype(np.float32)
    # applying it twice gives 32 x; rotated dot products are 32 times the originals (exact here)
    assert np.array_equal(Q.hadamard32(Q.hadamard32(q)), 32 * q)
    assert np.array_equal(Q.hadamard32(q).astype(np.float64) @ Q.hadamard32(k).astype(np.float64).T,
                          32 * (q.astype(np.float64) @ k.astype(np.float64).T))


def test_hadamard32_spreads_an_outlier_channel():
    # a lone channel of 8 becomes +-8 in every element of its block (row j of H),
    # and the MX exponent of the rotated block follows
    x = np.zeros((1, 64), np.float32)
    x[0, 37] = 8.0
    y = Q.hadamard32(x)
    H = _sylvester(32)
    assert np.array_equal(y[0, :32], np.zeros(32, np.float32))
    assert np.array_equal(y[0, 32:], (8.0 * H[:, 5]).astype(np.float32))
    codes, e8 = Q.quant_mxfp4(x, hadamard=True)
    assert e8.tolist() == [[0, 128]]         # block 1: amax 8 -> e = 3 - 2 = 1
    assert np.array_equal(Q.dequant_mxfp4(codes, e8)[0, 32:], y[0, 32:].astype(np.float64))
