"""Greedy block verification for parallel block drafting.

Follows the DFlash page (molayo1419.me, "How DFlash uses block diffusion to
remove the speculative-decoding bottleneck"), section "What DFlash does
differently", steps 3 and 4: the drafter fills a whole block of masked
positions in one pass, the target checks the block, accepted tokens are kept
and the first rejected one starts a new drafting cycle.  Under greedy
decoding a drafted token is accepted iff it equals the target's argmax, so
the accepted length is the length of the longest matching prefix.

Pinned by tests/test_oracle_verify.py (constructed targets whose first
mismatch position is known).
"""
from __future__ import annotations

import numpy as np


def verify_prefix(draft: np.ndarray, target: np.ndarray) -> np.ndarray:
    draft = np.asarray(draft)
    target = np.asarray(target)
    B, L = draft.shape
    out = np.full(B, L, np.int64)
    for b in range(B):
        for j in range(L):
            if draft[b, j] != target[b, j]:
                out[b] = j
                break
    return out
