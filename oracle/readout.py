"""Single-pass structured read: per-slot probabilities over the allowed choices.

Follows the single-pass-reads page ("DiffusionGemma's execution path merged",
portfolio.ywsung.com), section on answer slots: a fixed answer template
leaves one empty slot per question, one denoise pass over that canvas gives,
for every slot, the probability of each allowed choice.

Per slot with allowed ids a_0..a_{n-1}: q_j = exp(x_{a_j} - max) / sum_t exp(x_{a_t} - max),
x = logits / T, and the slot's answer is the first allowed id attaining the
largest logit.  (This equals the full-vocabulary softmax renormalised over
the allowed ids: the partition function cancels.)

Pinned by tests/test_oracle_readout.py: sum q = 1 and equality with the
renormalised full softmax of oracle.sampler.probabilities.
"""
from __future__ import annotations

import numpy as np


def allowed_probs(slot_logits: np.ndarray, offsets: np.ndarray, ids: np.ndarray, temperature: float = 1.0):
    """slot_logits [n_slots, V]; CSR (offsets [n_slots+1], ids) -> (q [len(ids)], answer [n_slots], gap [n_slots])."""
    n_slots = slot_logits.shape[0]
    q = np.zeros(ids.size)
    ans = np.zeros(n_slots, np.int64)
    gap = np.full(n_slots, np.inf)
    for s in range(n_slots):
        a = ids[offsets[s]:offsets[s + 1]]
        x = np.asarray(slot_logits[s, a], np.float64) / float(temperature)
        e = np.exp(x - np.max(x))
        q[offsets[s]:offsets[s + 1]] = e / np.sum(e)
        j = int(np.argmax(x))
        ans[s] = int(a[j])
        if a.size > 1:
            gap[s] = float(x[j] - np.max(np.delete(x, j)))
    return q, ans, gap
