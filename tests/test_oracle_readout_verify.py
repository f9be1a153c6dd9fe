"""Pins for oracle.readout (allowed-choice probabilities) and oracle.verify (greedy prefix)."""
import numpy as np

from oracle import readout, sampler, verify


def test_allowed_probs_is_renormalised_softmax():
    rng = np.random.default_rng(0)
    L = rng.normal(0, 3, (5, 2000))
    counts = [2, 3, 4, 5, 2]
    ids = np.concatenate([rng.choice(2000, c, replace=False) for c in counts])
    off = np.concatenate([[0], np.cumsum(counts)])
    q, ans, _ = readout.allowed_probs(L, off, ids)
    for s in range(5):
        a = ids[off[s]:off[s + 1]]
        p = sampler.probabilities(L[s], 1.0)[a]
        np.testing.assert_allclose(q[off[s]:off[s + 1]], p / p.sum(), rtol=1e-12)
        assert abs(q[off[s]:off[s + 1]].sum() - 1) < 1e-12
        assert ans[s] == a[np.argmax(L[s, a])]


def test_allowed_ties_take_first_listed():
    L = np.zeros((1, 10))
    q, ans, gap = readout.allowed_probs(L, np.array([0, 3]), np.array([7, 2, 5]))
    assert ans[0] == 7 and np.allclose(q, 1 / 3) and gap[0] == 0


def test_verify_prefix_constructed():
    rng = np.random.default_rng(1)
    draft = rng.integers(0, 100, (200, 16))
    g = rng.geometric(0.2, 200) - 1                  # matches before the first mismatch
    target = draft.copy()
    for b in range(200):
        if g[b] < 16:
            target[b, g[b]] = (draft[b, g[b]] + 1 + rng.integers(0, 99)) % 100
            target[b, g[b] + 1:] = rng.integers(0, 100, 15 - g[b])
    assert np.array_equal(verify.verify_prefix(draft, target), np.minimum(g, 16))
