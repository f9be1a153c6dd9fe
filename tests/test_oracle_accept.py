"""Pins for oracle.accept: brute-force subset enumeration on tiny canvases."""
import itertools

import numpy as np
import pytest

from oracle import accept, philox


def brute_force_accept_set(H, budget):
    """Among all subsets with total entropy <= budget, the largest; ties between equally large
    subsets go to the one whose ascending (H, pos) list is lexicographically smallest."""
    C = len(H)
    best = None
    for r in range(C, -1, -1):
        cands = []
        for sub in itertools.combinations(range(C), r):
            if sum(float(H[i]) for i in sub) <= budget:
                cands.append(sorted((float(H[i]), i) for i in sub))
        if cands:
            best = min(cands)
            break
    return sorted(i for _, i in best)


@pytest.mark.parametrize("seed", range(40))
def test_accept_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    C = int(rng.integers(1, 11))
    # coarse values create exact entropy ties; fp32 like the kernel's inputs
    H = (rng.integers(0, 6, C) * 0.5 + (rng.random(C) < 0.3) * rng.random(C)).astype(np.float32)
    budget = float(rng.choice([0.0, 0.5, 1.0, 2.0, 3.7, 100.0]))
    sample = rng.integers(0, 1000, (1, C))
    canvas = rng.integers(0, 1000, (1, C))
    o = accept.entropy_accept(H[None, :], sample, canvas, budget, [7], [3], 1000)
    acc = sorted(np.nonzero(o.accept[0])[0].tolist())
    assert acc == brute_force_accept_set(H, budget)
    assert o.n_accept[0] == len(acc)
    noise = philox.random_tokens(7, 3, np.arange(C), 1000, philox.RENOISE)
    for i in range(C):
        assert o.canvas[0, i] == (sample[0, i] if i in acc else noise[i])


def test_accept_special_cases():
    H = np.array([[0.5, 0.1, 0.1, 2.0]], np.float32)
    s = np.array([[10, 11, 12, 13]])
    c = np.zeros((1, 4), np.int64)
    assert accept.entropy_accept(H, s, c, 0.0, [1], [0], 50).n_accept[0] == 0
    o = accept.entropy_accept(H, s, c, float(H.astype(np.float64).sum()), [1], [0], 50)
    assert o.n_accept[0] == 4 and np.array_equal(o.canvas[0], s[0])          # equality accepts
    o = accept.entropy_accept(H, s, c, 0.2, [1], [0], 50)     # fp32 0.1 is just above 0.1: 0.1f + 0.1f > 0.2
    assert np.float64(np.float32(0.1)) * 2 > 0.2 and o.n_accept[0] == 1
    o = accept.entropy_accept(H, s, c, 0.15, [1], [0], 50)
    assert o.n_accept[0] == 1 and o.accept[0, 1] == 1                         # tie -> lower position
    Z = np.zeros((2, 5), np.float32)
    o = accept.entropy_accept(Z, np.ones((2, 5), int), np.zeros((2, 5)), 0.0, [1, 2], [0, 0], 9, active=[1, 0])
    assert o.n_accept.tolist() == [5, 0] and o.canvas[1].tolist() == [0] * 5  # inactive untouched
