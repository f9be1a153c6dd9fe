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
      stream GUMBEL       = 0 : one word per block of 16 vocabulary ids (the block level of the
                                 two-level Gumbel-max draw): block b uses word (b >> 7) & 3 of
                                 counter c0 = 128 * (b >> 9) + (b & 127)
      stream RENOISE      = 1 : c0 = 0, word 0
      stream INIT         = 2 : c0 = 0, word 0
      stream GUMBEL_INNER = 3 : element level, inside the winning block: vocabulary element i
                                 uses word i & 3 of counter c0 = i >> 2
  step is the request's global step counter, never reset between blocks.
  The block map (b -> c0, word) is a bijection onto (counter, word) pairs, so every block of a
  position gets its own Philox output word and the block noise values are independent; the four
  blocks p, p + 128, p + 256, p + 384 of each run of 512 blocks share one counter (words 0..3),
  so a pass that reads the row in runs of 128 blocks draws the noise of four blocks with one
  Philox call.  Any bijection gives the same law of the draw; this one is fixed so that the two
  sides of a parity test draw identical noise.

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
GUMBEL_INNER = 3
GUMBEL_BLOCK = 16   # vocabulary ids per block of the two-level Gumbel-max draw


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


def _words(seed: int, pos: int, step: int, c0, word, stream: int) -> np.ndarray:
    c0 = np.asarray(c0, dtype=np.int64)
    ctr = np.zeros(c0.shape + (4,), np.uint32)
    ctr[..., 0] = c0.astype(np.uint32)
    ctr[..., 1] = np.uint32(pos)
    ctr[..., 2] = np.uint32(step & 0xFFFFFFFF)
    ctr[..., 3] = np.uint32(stream)
    out = philox4x32_10(ctr, seed_key(seed))
    return np.take_along_axis(out, np.asarray(word, np.int64)[..., None], axis=-1)[..., 0]


def block_counter_word(b):
    """(c0, word) of block b in stream GUMBEL."""
    b = np.asarray(b, dtype=np.int64)
    return 128 * (b >> 9) + (b & 127), (b >> 7) & 3


def block_gumbels(seed: int, pos: int, step: int, nblocks: int) -> np.ndarray:
    """Gumbel noise G_b, b = 0..nblocks-1, of the blocks of one canvas position (stream GUMBEL)."""
    c0, w = block_counter_word(np.arange(nblocks))
    return gumbel_from_word(_words(seed, pos, step, c0, w, GUMBEL))


def inner_gumbels(seed: int, pos: int, step: int, lo: int, hi: int) -> np.ndarray:
    """Gumbel noise g_i, i = lo..hi-1, of vocabulary elements (stream GUMBEL_INNER)."""
    i = np.arange(lo, hi, dtype=np.int64)
    return gumbel_from_word(_words(seed, pos, step, i >> 2, i & 3, GUMBEL_INNER))


def random_tokens(seed: int, step: int, positions, V: int, stream: int) -> np.ndarray:
    """One random token id per position from word 0 of Philox(key, (0, pos, step, stream))."""
    positions = np.asarray(positions, dtype=np.int64)
    ctr = np.zeros(positions.shape + (4,), np.uint32)
    ctr[..., 1] = positions.astype(np.uint32)
    ctr[..., 2] = np.uint32(step & 0xFFFFFFFF)
    ctr[..., 3] = np.uint32(stream)
    words = philox4x32_10(ctr, seed_key(seed))[..., 0]
    return token_from_word(words, V)
