"""Element and scale codecs used by the oracle.  TEST INFRASTRUCTURE ONLY.

Formats (the pages name them; the bit layouts are the OCP 8-bit floating
point and OCP Microscaling (MX) v1.0 definitions):

* E2M1 ("FP4"): 1 sign bit (bit 3), 2 exponent bits (bias 1), 1 mantissa bit.
  Magnitudes of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Used for the NVFP4
  Q/K payloads, the Direct-P probability codes and MXFP4 V
  ("Hardware-Aware FP4 FlashAttention-4", summary page, "What the paper found").
* E4M3 (the "fn" variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
  no infinities, 0x7F/0xFF are NaN, largest finite 448, subnormals down to
  2**-9.  Used for the NVFP4 block scales, FP8 V and FP8 P.
* E5M2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits, largest finite
  57344, subnormals down to 2**-16; 0x7C is infinity and 0x7D..0x7F NaN.  Used
  for the output gradient dO of the backward (summary page, "What the paper
  found": FP8 gradient operands, with E5M2 output gradients).
* E8M0: an unsigned biased exponent, value 2**(k-127) for k in 0..254, 255 is
  NaN.  Used for the per-32-element MX scales.

Rounding reading (the pages fix none): every encoder rounds to nearest with
ties to the even code, and saturates to the largest finite magnitude (6 for
E2M1, 448 for E4M3).  The sign of the input is kept, so a negative input that
rounds to zero gives negative zero (E2M1 code 8, E4M3 code 0x80).
"""

import numpy as np

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0
E5M2_MAX = 57344.0


def _round_to_minifloat(a, mbits, emin):
    """Round non-negative float64 magnitudes ``a`` to the grid of a minifloat
    with ``mbits`` mantissa bits and smallest normal exponent ``emin``
    (round to nearest, ties to even).  No saturation here."""
    a = np.asarray(a, dtype=np.float64)
    _, k = np.frexp(a)                      # a = f * 2**k, f in [0.5, 1)
    e = np.maximum(k.astype(np.int64) - 1, emin)
    e = np.where(a == 0, emin, e)
    q = np.ldexp(1.0, (e - mbits).astype(np.int64))
    return np.rint(a / q) * q               # a / q is exact (power-of-two divide)


def e2m1_decode(codes):
    """E2M1 codes (uint8, low 4 bits used) -> float64 values."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_encode(x):
    """Real values -> E2M1 codes (uint8), round-to-nearest-even, saturating."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    r = np.minimum(_round_to_minifloat(a, 1, 0), E2M1_MAX)
    code = np.searchsorted(E2M1_MAGNITUDES, r).astype(np.uint8)
    return np.where(np.signbit(x), code | 8, code).astype(np.uint8)


def e4m3_decode(codes):
    """E4M3 (fn) codes -> float64 values; 0x7F / 0xFF decode to NaN."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(x):
    """Real values -> E4M3 (fn) codes, round-to-nearest-even, saturating to 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    r = np.minimum(_round_to_minifloat(a, 3, -6), E4M3_MAX)
    _, k = np.frexp(r)
    e = k.astype(np.int64) - 1
    sub = r < 2.0 ** -6
    mant = np.where(sub, 0, np.rint((r / np.ldexp(1.0, np.where(sub, 0, e)) - 1.0) * 8.0))
    code = np.where(sub, np.rint(r * 2.0 ** 9), ((e + 7) << 3) + mant).astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def e5m2_decode(codes):
    """E5M2 codes -> float64 values (0x7C/0xFC are +-inf, 0x7D..0x7F NaN)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    s = c >> 7
    e = (c >> 2) & 0x1F
    m = c & 3
    mag = np.where(e == 0, m * 2.0 ** -16, (1.0 + m / 4.0) * np.ldexp(1.0, e - 15))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def e5m2_encode(x):
    """Real values -> E5M2 codes, round-to-nearest-even, saturating to 57344."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    r = np.minimum(_round_to_minifloat(a, 2, -14), E5M2_MAX)
    _, k = np.frexp(r)
    e = k.astype(np.int64) - 1
    sub = r < 2.0 ** -14
    mant = np.where(sub, 0, np.rint((r / np.ldexp(1.0, np.where(sub, 0, e)) - 1.0) * 4.0))
    code = np.where(sub, np.rint(r * 2.0 ** 16), ((e + 15) << 2) + mant).astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def e8m0_decode(codes):
    """E8M0 scale bytes -> float64 values 2**(k-127); 255 decodes to NaN."""
    k = np.asarray(codes).astype(np.int64) & 0xFF
    v = np.ldexp(1.0, k - 127)
    return np.where(k == 255, np.nan, v)


def e8m0_encode_exponent(e):
    """Integer exponents in [-127, 127] -> E8M0 bytes (k = e + 127)."""
    e = np.asarray(e, dtype=np.int64)
    if np.any(e < -127) or np.any(e > 127):
        raise ValueError("E8M0 exponent out of range")
    return (e + 127).astype(np.uint8)


def pack_nibbles(codes):
    """uint8 codes (last axis even length) -> bytes, element 2k in the low
    nibble and element 2k+1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed):
    """Inverse of :func:`pack_nibbles`."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
