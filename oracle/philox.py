"""Philox4x32-10 counter-based generator and the denoise step's noise mappings.

Source of the generator: Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
as easy as 1, 2, 3" (SC'11), the Philox-4x32 bijection with 10 rounds.  The
pages ask only for noise keyed by (seed, step, position) [DiffusionGemma page,
section "DiffusionGemmaModelState and DiffusionSampler", the denoise case:
Gumbel candidate per position, random-token renoising]; the keying and the
mappings below are this library's reading of that (listed as readings in the
design notes).

Keying
  key     = (seed & 0xffffffff, seed >> 32)           -- one 64-bit seed per request
  counter = (c0, pos, step, stream)
      stream GUMBEL  = 0 : c0 = i >> 2, vocabulary element i uses word i & 3
      stream RENOISE = 1 : c0 = 0, word 0
      stream INIT    = 2 : c0 = 0, word 0
  step is the request's global step counter, never reset between blocks.

Mappings
  uniform(w) = (2 * (w >> 9) + 1) * 2**-24         in (0, 1); exact in fp32
  gumbel(w)  = -ln(-ln(uniform(w)))
  token(w, V) = (w * V) >> 32                      (multiply-high)

Pinned by: tests/test_oracle_philox.py (cross-check against two independently
written, installed Philox4x32-10 implementations run as black boxes, plus
distribution tests of the mappings).
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint32(0x9E3779B9)
W1 = np.uint32(0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)

GUMBEL = 0
RENOISE = 1
INIT = 2


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds.

    ctr: uint32 array [..., 4]; key: uint32 array [..., 2] (broadcastable).
    Returns the four output words, uint32 [..., 4].
    Each round multiplies words 0 and 2 by the two Philox constants, swaps the
    product halves into place and XORs the high halves with words 1, 3 and the
    key; the key is bumped by the two Weyl constants between rounds.
    """
    ctr = np.asarray(ctr, dtype=np.uint32)
    key = np.asarray(key, dtype=np.uint32)
    shape = np.broadcast_shapes(ctr.shape[:-1], key.shape[:-1])
    c = [np.broadcast_to(ctr[..., j], shape).astype(np.uint64) for j in range(4)]
    k0 = np.broadcast_to(key[..., 0], shape).astype(np.uint32).copy()
    k1 = np.broadcast_to(key[..., 1], shape).astype(np.uint32).copy()
    with np.errstate(over="ignore"):
        for rnd in range(10):
            if rnd:
                k0 = k0 + W0
                k1 = k1 + W1
            p0 = M0 * c[0]
            p1 = M1 * c[2]
            hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
            hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
            c = [hi1 ^ c[1] ^ k0.astype(np.uint64),
                 lo1,
                 hi0 ^ c[3] ^ k1.astype(np.uint64),
                 lo0]
    return np.stack([x.astype(np.uint32) for x in c], axis=-1)


def seed_key(seed) -> np.ndarray:
    s = np.asarray(seed, dtype=np.uint64)
    return np.stack([(s & MASK32).astype(np.uint32), (s >> np.uint64(32)).astype(np.uint32)], axis=-1)


def uniform_from_word(w) -> np.ndarray:
    """(2*(w>>9)+1) * 2^-24 as float64 (exactly representable in fp32)."""
    w = np.asarray(w, dtype=np.uint32)
    return ((w >> np.uint32(9)).astype(np.float64) * 2.0 + 1.0) * 2.0 ** -24


def gumbel_from_word(w) -> np.ndarray:
    return -np.log(-np.log(uniform_from_word(w)))


def token_from_word(w, V: int) -> np.ndarray:
    return ((np.asarray(w, dtype=np.uint64) * np.uint64(V)) >> np.uint64(32)).astype(np.int64)


def gumbel_row(seed: int, pos: int, step: int, V: int) -> np.ndarray:
    """Gumbel noise g_i, i = 0..V-1, for one canvas position (stream GUMBEL)."""
    n = (V + 3) // 4
    ctr = np.zeros((n, 4), np.uint32)
    ctr[:, 0] = np.arange(n, dtype=np.uint32)
    ctr[:, 1] = np.uint32(pos)
    ctr[:, 2] = np.uint32(step & 0xFFFFFFFF)
    ctr[:, 3] = np.uint32(GUMBEL)
    words = philox4x32_10(ctr, seed_key(seed)).reshape(-1)[:V]
    return gumbel_from_word(words)


def random_tokens(seed: int, step: int, positions, V: int, stream: int) -> np.ndarray:
    """One random token id per position from word 0 of Philox(key, (0, pos, step, stream))."""
    positions = np.asarray(positions, dtype=np.int64)
    ctr = np.zeros(positions.shape + (4,), np.uint32)
    ctr[..., 1] = positions.astype(np.uint32)
    ctr[..., 2] = np.uint32(step & 0xFFFFFFFF)
    ctr[..., 3] = np.uint32(stream)
    words = philox4x32_10(ctr, seed_key(seed))[..., 0]
    return token_from_word(words, V)
