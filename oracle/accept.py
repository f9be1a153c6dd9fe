"""Entropy-budget acceptance and random-token renoising.

Follows the DiffusionGemma/vLLM page, section "Entropy-based denoising": the
positions of a canvas are visited from most to least confident (lowest to
highest entropy) and accepted as long as the running entropy total stays
within the budget; every other position is replaced by a fresh random token
for the next step.  The denoise case of "DiffusionGemmaModelState and
DiffusionSampler" says the accepted positions keep the Gumbel candidate.

Readings: ties in entropy are ordered by position; a running total equal to
the budget is accepted; zero accepted positions is allowed; the running total
is an fp64 sum of the (fp32) entropies; renoise tokens come from the Philox
RENOISE stream at the request's global step.

Pinned by tests/test_oracle_accept.py: brute-force enumeration of all subsets
of tiny canvases (the accepted set is the maximum-cardinality subset within
the budget whose sorted (H, pos) list is lexicographically smallest), plus
special cases (budget 0, budget >= total, all-equal entropies).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import philox


@dataclass
class AcceptOut:
    canvas: np.ndarray     # int64 [B, C]
    accept: np.ndarray     # uint8 [B, C]
    n_accept: np.ndarray   # int64 [B]
    budget_gap: np.ndarray  # float64 [B]: min |running total - budget| at the cut (near-tie measure)


def accept_order(H_row: np.ndarray) -> np.ndarray:
    """Positions sorted by (entropy, position) ascending."""
    H_row = np.asarray(H_row, dtype=np.float64)
    return np.lexsort((np.arange(H_row.size), H_row))


def n_within_budget(H_row: np.ndarray, budget: float):
    order = accept_order(H_row)
    cs = np.cumsum(np.asarray(H_row, dtype=np.float64)[order])
    n = int(np.sum(cs <= budget))
    gaps = []
    if n > 0:
        gaps.append(abs(cs[n - 1] - budget))
    if n < cs.size:
        gaps.append(abs(cs[n] - budget))
    return order, n, (min(gaps) if gaps else np.inf)


def entropy_accept(entropy: np.ndarray, sample: np.ndarray, canvas: np.ndarray, budget: float,
                   seeds, steps, V: int, active=None) -> AcceptOut:
    entropy = np.asarray(entropy, dtype=np.float64)
    B, C = entropy.shape
    canvas = np.array(canvas, dtype=np.int64, copy=True)
    accept = np.zeros((B, C), np.uint8)
    n_acc = np.zeros(B, np.int64)
    gap = np.full(B, np.inf)
    for b in range(B):
        if active is not None and not active[b]:
            continue
        order, n, g = n_within_budget(entropy[b], budget)
        n_acc[b] = n
        gap[b] = g
        noise = philox.random_tokens(int(seeds[b]), int(steps[b]), np.arange(C), V, philox.RENOISE)
        new = noise.copy()
        acc = order[:n]
        new[acc] = np.asarray(sample[b], dtype=np.int64)[acc]
        accept[b, acc] = 1
        canvas[b] = new
    return AcceptOut(canvas=canvas, accept=accept, n_accept=n_acc, budget_gap=gap)
