"""Pins of the oracle's codecs against closed forms and torch's float8 dtypes."""

import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e2m1_decode_closed_form():
    # OCP E2M1: bias 1; exponent field 0 is subnormal (0 or 0.5).
    expect = []
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        expect.append(-mag if s else mag)
    got = F.e2m1_decode(np.arange(16))
    np.testing.assert_array_equal(got, np.array(expect))
    np.testing.assert_array_equal(got[:8], [0, 0.5, 1, 1.5, 2, 3, 4, 6])


def _brute_e2m1(x):
    """Nearest E2M1 magnitude by distance; ties go to the even code; above 6
    saturates.  Independent of the oracle's exponent/rint route."""
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    out = []
    for v in x:
        a = abs(v)
        if a >= 6:
            c = 7
        else:
            d = np.abs(mags - a)
            best = np.flatnonzero(d == d.min())
            c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out.append(c | (8 if np.signbit(v) else 0))
    return np.array(out, np.uint8)


def test_e2m1_encode_bruteforce():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    exact = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    grid = np.linspace(-8, 8, 4097)
    eps = [np.nextafter(m, 0) for m in mids] + [np.nextafter(m, 10) for m in mids]
    x = np.concatenate([grid, mids, exact, eps, -np.array(mids), [7, 100, 1e30, -1e30]])
    np.testing.assert_array_equal(F.e2m1_encode(x), _brute_e2m1(x))


def test_e2m1_ties_to_even_code():
    # midpoint -> even code: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2, 2.5->2, 3.5->4, 5->4
    got = F.e2m1_decode(F.e2m1_encode([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]))
    np.testing.assert_array_equal(got, [0, 1, 1, 2, 2, 4, 4])


def test_e2m1_sign_and_negative_zero():
    assert F.e2m1_encode([-0.0])[0] == 8
    assert F.e2m1_encode([-0.1])[0] == 8
    assert F.e2m1_encode([-6.5])[0] == 15


def _all_finite_bf16():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.bfloat16)
    x = x[torch.isfinite(x)]
    return x


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(codes.numpy())
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_e4m3_encode_matches_torch_on_all_bf16():
    # torch's cast rounds to nearest even but does not saturate (NaN past 464),
    # so compare where it is finite and check saturation separately.
    x = _all_finite_bf16()
    ref = x.to(torch.float8_e4m3fn)
    finite = torch.isfinite(ref.to(torch.float32))
    got = F.e4m3_encode(x.to(torch.float32).numpy())
    np.testing.assert_array_equal(got[finite.numpy()], ref.view(torch.uint8).numpy()[finite.numpy()])
    big = (~finite).numpy()
    xs = x.to(torch.float32).numpy()[big]
    assert np.all(np.abs(xs) >= 464)
    np.testing.assert_array_equal(got[big], np.where(xs < 0, 0xFE, 0x7E).astype(np.uint8))


def test_e4m3_encode_matches_torch_random_f32():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp2(rng.uniform(-14, 9, 200000))).astype(np.float32)
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(F.e4m3_encode(x), ref)


def test_e8m0_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = F.e8m0_decode(codes.numpy())
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_nibble_order():
    codes = np.array([[1, 2, 3, 4, 15, 0]], np.uint8)
    packed = F.pack_nibbles(codes)
    np.testing.assert_array_equal(packed, [[0x21, 0x43, 0x0F]])
    np.testing.assert_array_equal(F.unpack_nibbles(packed), codes)


def test_e8m0_exponent_range():
    assert F.e8m0_encode_exponent([-127, 0, 127]).tolist() == [0, 127, 254]
    with pytest.raises(ValueError):
        F.e8m0_encode_exponent([128])


def test_e5m2_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    got = F.e5m2_decode(codes.numpy())
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_e5m2_encode_matches_torch_on_all_bf16():
    # torch's cast rounds to nearest even; past 61440 it gives infinity, where
    # the oracle saturates to 57344
    x = _all_finite_bf16()
    ref = x.to(torch.float8_e5m2)
    finite = torch.isfinite(ref.to(torch.float32))
    got = F.e5m2_encode(x.to(torch.float32).numpy())
    np.testing.assert_array_equal(got[finite.numpy()], ref.view(torch.uint8).numpy()[finite.numpy()])
    big = (~finite).numpy()
    xs = x.to(torch.float32).numpy()[big]
    assert np.all(np.abs(xs) >= 61440)
    np.testing.assert_array_equal(got[big], np.where(xs < 0, 0xFB, 0x7B).astype(np.uint8))


def test_e5m2_encode_matches_torch_random_f32():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * np.exp2(rng.uniform(-20, 15, 200000))).astype(np.float32)
    x = x[np.abs(x) < 61440]
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    np.testing.assert_array_equal(F.e5m2_encode(x), ref)
