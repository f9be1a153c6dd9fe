"""OCP 8-bit floating point E4M3 (the "e4m3fn" encoding) decoded to float64.

Test infrastructure: the oracle of the E4M3 embedding-table variant of self-conditioning
(DiffusionGemma/vLLM page, section on quantised checkpoints: the model ships FP8 weights; here the
embedding table E is stored as E4M3 codes times one scale).  Encoding per the OCP 8-bit floating
point specification: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa; exponent 0 is
subnormal (m / 8 * 2^-6); exponent 15 with mantissa 7 is NaN; there are no infinities, so the
largest finite value is 1.75 * 2^8 = 448.

Pinned by tests/test_oracle_fp8.py: the specification's landmark values (smallest subnormal,
largest subnormal, smallest normal, one, largest finite, NaN, signed zero), strict monotonicity
over the finite codes, and torch's own float8_e4m3fn conversion of all 256 codes (an independent
library implementation).
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
