"""Pins for oracle.admission (deficit token-budget admission).

* a hand-worked trace of the page's rule (tests/golden/deficit_trace.txt);
* a closed form: prefill i starts owing at s_i = max(arrival_i, admitted_{i-1} + 1) and is admitted
  at the first t >= s_i whose leftover budget summed over s_i .. t reaches its size (numpy cumsum
  and searchsorted, no iteration state);
* the properties the page states: decode work first, prefills whole, and no starvation: with at
  least r > 0 tokens left over every iteration a prefill of size P waits at most ceil(P / r)
  iterations once it is at the head of the queue.
"""
import os

import numpy as np
import pytest

from oracle import admission

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "deficit_trace.txt")


def read_trace():
    budget, arrivals, iters = None, [], []
    with open(GOLDEN) as f:
        for line in f:
            tok = line.split()
            if not tok or tok[0].startswith("#"):
                continue
            if tok[0] == "budget":
                budget = int(tok[1])
            elif tok[0] == "arrival":
                arrivals.append((int(tok[2]), int(tok[3])))
            elif tok[0] == "iter":
                iters.append((int(tok[2]), None if tok[3] == "-" else int(tok[3]), int(tok[4]), int(tok[5])))
    return budget, arrivals, iters


def test_hand_worked_trace():
    budget, arrivals, iters = read_trace()
    tr = admission.simulate(budget, [it[0] for it in iters], arrivals)
    assert tr.admitted == [[] if it[1] is None else [it[1]] for it in iters]
    assert tr.tokens == [it[2] for it in iters]
    assert tr.deficit == [it[3] for it in iters]


def closed_form(budget, decode, arrivals):
    """Admission iteration of every prefill (or -1), from prefix sums of the leftover budget."""
    remain = budget - np.asarray(decode, np.int64)
    out = []
    prev = -1
    for t_arr, size in arrivals:
        s = max(t_arr, prev + 1)
        if s >= len(remain):
            out.append(-1)
            prev = len(remain)
            continue
        csum = np.cumsum(remain[s:])
        # the running sum need not be monotone (remain may be negative): first index reaching size
        hit = np.nonzero(csum >= size)[0]
        t = s + int(hit[0]) if hit.size else -1
        out.append(t)
        prev = t if t >= 0 else len(remain)
    return out


def random_case(rng, n_iter=60, n_pf=12, budget=64):
    decode = rng.integers(0, budget + 16, n_iter)            # sometimes above the budget
    arr = np.sort(rng.integers(0, n_iter, n_pf))
    sizes = rng.integers(1, 4 * budget, n_pf)
    return budget, decode.tolist(), [(int(a), int(s)) for a, s in zip(arr, sizes)]


@pytest.mark.parametrize("seed", range(20))
def test_closed_form_of_admission_times(seed):
    budget, decode, arrivals = random_case(np.random.default_rng(seed))
    tr = admission.simulate(budget, decode, arrivals)
    when = [-1] * len(arrivals)
    for t, ids in enumerate(tr.admitted):
        for pid in ids:
            when[pid] = t
    assert when == closed_form(budget, decode, arrivals)


@pytest.mark.parametrize("seed", range(20))
def test_decode_first_and_whole_prefills(seed):
    budget, decode, arrivals = random_case(np.random.default_rng(100 + seed))
    tr = admission.simulate(budget, decode, arrivals)
    order = [pid for ids in tr.admitted for pid in ids]
    assert order == sorted(order)                               # first come, first served
    for t, ids in enumerate(tr.admitted):
        assert len(ids) <= 1
        assert tr.tokens[t] == decode[t] + sum(arrivals[p][1] for p in ids)   # decode never cut, prefill whole


@pytest.mark.parametrize("r", [1, 5, 17])
def test_no_starvation_bound(r):
    rng = np.random.default_rng(r)
    budget = 40
    n_iter = 400
    decode = (budget - r - rng.integers(0, 3, n_iter)).tolist()    # leftover >= r every iteration
    arrivals = [(0, int(s)) for s in rng.integers(1, 200, 8)]
    tr = admission.simulate(budget, decode, arrivals)
    when = {pid: t for t, ids in enumerate(tr.admitted) for pid in ids}
    assert len(when) == len(arrivals)
    prev = -1
    for pid, (t_arr, size) in enumerate(arrivals):
        head = max(t_arr, prev + 1)
        assert when[pid] - head + 1 <= -(-size // r)
        prev = when[pid]


def test_without_carry_a_large_prefill_never_enters():
    """The page's reason for carrying the deficit: a prefill larger than every iteration's leftover
    budget enters only because D accumulates."""
    budget, decode = 10, [7] * 50
    tr = admission.simulate(budget, decode, [(0, 25)])
    assert [t for t, ids in enumerate(tr.admitted) if ids] == [8]   # 3 per iteration: 9 iterations
    # with D pinned at 0 the admission test 3 + 0 >= 25 never holds
    assert all(admission.admit(budget, 7, [25], 0)[0] == 0 for _ in range(50))
