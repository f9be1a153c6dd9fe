"""OCP 8-bit floating point E4M3 (the "e4m3fn" encoding) decoded to float64.

Test infrastructure: the oracle of the E4M3 embedding-table variant of self-conditioning
(DiffusionGemma/vLLM page, section on quantised checkpoints: the model ships FP8 weights; here the
embedding table E is stored as E4M3 codes times one scale).  Encoding per the OCP 8-bit floating
point specification: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa; exponent 0 is
subnormal (m / 8 * 2^-6); exponent 15 with mantissa 7 is NaN; there are no infinities, so the
largest finite value is 1.75 * 2^8 = 448.

Encoding (used for the E4M3 paged KV cache, where appended keys and values are quantised): round
to the nearest finite E4M3 value, ties to the even code (mantissa bit 0 clear), magnitudes above
448 saturate to +-448 (the specification's saturating conversion), NaN stays NaN.

Pinned by tests/test_oracle_fp8.py: the specification's landmark values (smallest subnormal,
largest subnormal, smallest normal, one, largest finite, NaN, signed zero), strict monotonicity
over the finite codes, torch's own float8_e4m3fn conversion of all 256 codes (an independent
library implementation); for encoding, the round trip of every finite code, hand-picked midpoints
(ties to even), saturation, and torch's round-to-nearest conversion on random in-range values.
"""
from __future__ import annotations

import numpy as np


def decode_e4m3(codes) -> np.ndarray:
    """uint8 codes (any shape) -> float64 values."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m / 8.0 * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    v = sign * np.where(e == 0, sub, nrm)
    return np.where((e == 15) & (m == 7), np.nan, v)


def decode_table(codes, scale: float) -> np.ndarray:
    """A scaled E4M3 table: scale * decode(codes) in float64."""
    return float(scale) * decode_e4m3(codes)


_POS = None


def _positive_values():
    global _POS
    if _POS is None:
        _POS = decode_e4m3(np.arange(0x00, 0x7F, dtype=np.uint8))   # codes 0 .. 126: 0 .. 448, increasing
    return _POS


def encode_e4m3(x) -> np.ndarray:
    """float values (any shape) -> uint8 E4M3 codes, round to nearest, ties to even, saturating."""
    x = np.asarray(x, dtype=np.float64)
    pos = _positive_values()
    a = np.minimum(np.abs(x), pos[-1])
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, pos.size - 1)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - pos[lo], pos[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == pos[hi], hi, code)
    out = (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), out)
