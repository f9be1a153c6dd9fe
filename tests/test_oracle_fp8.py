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
