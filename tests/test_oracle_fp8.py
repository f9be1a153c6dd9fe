"""Pins for oracle.fp8 (OCP E4M3 decoding)."""
import numpy as np

from oracle import fp8


def test_specification_landmarks():
    d = lambda c: float(fp8.decode_e4m3(np.uint8(c)))
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert d(0x01) == 2.0 ** -9                     # smallest subnormal
    assert d(0x07) == 0.875 * 2.0 ** -6             # largest subnormal
    assert d(0x08) == 2.0 ** -6                     # smallest normal
    assert d(0x38) == 1.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0   # largest finite
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x3F) == 1.875 and d(0x40) == 2.0


def test_monotone_over_finite_codes():
    pos = fp8.decode_e4m3(np.arange(0x00, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = fp8.decode_e4m3(np.arange(0x80, 0xFF, dtype=np.uint8))
    np.testing.assert_array_equal(neg, -pos)


def test_matches_torch_float8_e4m3fn():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.decode_e4m3(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_encode_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = fp8.decode_e4m3(codes)
    got = fp8.encode_e4m3(vals)
    # +0 and -0 both decode to zero; their codes keep the sign
    np.testing.assert_array_equal(got, codes)


def test_encode_ties_to_even_and_saturation():
    e = lambda v: int(fp8.encode_e4m3(np.float64(v)))
    assert e(1.0625) == 0x38            # between 1.0 (0x38) and 1.125 (0x39): even code
    assert e(1.1875) == 0x3A            # between 1.125 (0x39) and 1.25 (0x3A): even code
    assert e(1.07) == 0x39 and e(1.06) == 0x38
    assert e(2.0 ** -10) == 0x00 and e(1.5 * 2.0 ** -9) == 0x02   # ties at the subnormal end
    assert e(2.0 ** -10 * 1.01) == 0x01
    assert e(448.0) == 0x7E and e(464.0) == 0x7E and e(1e6) == 0x7E and e(-1e6) == 0xFE
    assert e(-1.0) == 0xB8 and np.isnan(fp8.decode_e4m3(fp8.encode_e4m3(np.nan)))


def test_encode_matches_torch_round_to_nearest_in_range():
    import torch
    x = np.random.default_rng(0).normal(0, 40, 20000)
    x = x[np.abs(x) < 440]
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(fp8.encode_e4m3(x.astype(np.float32).astype(np.float64)), ref)
