"""Pins for oracle.converged: hand-built histories with known outcomes."""
import numpy as np

from oracle import converged as cv
from oracle import philox


def fresh(B, C):
    return cv.LoopState(canvas=np.zeros((B, C), np.int64), prev_argmax=np.zeros((B, C), np.int64),
                        unchanged=np.zeros(B, np.int64), step_in_block=np.full(B, -1, np.int64),
                        step_global=np.zeros(B, np.int64), sc_on=np.zeros(B, np.uint8))


def run(history, H, k, tau, max_steps, C=4, V=100, seed=9):
    st = fresh(1, C)
    cv.converged(np.zeros((1, C)), np.zeros((1, C)), st, k, tau, max_steps, [seed], V)  # prefill
    for t, a in enumerate(history):
        o = cv.converged(np.asarray(a)[None, :], np.full((1, C), H), st, k, tau, max_steps, [seed], V)
        if o.committed[0]:
            return t, o, st
    return None, None, st


def test_prefill_case_random_canvas():
    st = fresh(2, 8)
    st.step_global[:] = [0, 5]
    o = cv.converged(np.zeros((2, 8)), np.zeros((2, 8)), st, 2, 0.5, 32, [3, 4], 1024)
    assert o.num_sampled.tolist() == [0, 0] and o.committed.tolist() == [0, 0]
    assert np.array_equal(st.canvas[0], philox.random_tokens(3, 0, np.arange(8), 1024, philox.INIT))
    assert np.array_equal(st.canvas[1], philox.random_tokens(4, 5, np.arange(8), 1024, philox.INIT))
    assert st.step_in_block.tolist() == [0, 0] and st.step_global.tolist() == [1, 6]


def test_constant_argmax_zero_entropy_commits_after_k_plus_1():
    for k in (1, 2, 3, 5):
        t, o, st = run([[1, 2, 3, 4]] * 40, 0.0, k, 0.5, 32)
        assert o.steps_used[0] == k + 1 and t == k
        assert o.out_tokens[0].tolist() == [1, 2, 3, 4] and o.num_sampled[0] == 4
        assert st.step_in_block[0] == 0 and st.unchanged[0] == 0 and st.sc_on[0] == 0
        g = st.step_global[0] - 1    # the restart canvas is drawn at the commit step's global step
        assert np.array_equal(st.canvas[0], philox.random_tokens(9, g, np.arange(4), 100, philox.INIT))


def test_alternating_argmax_runs_to_cap():
    hist = [[1, 2, 3, 4], [1, 2, 3, 5]] * 30
    t, o, _ = run(hist, 0.0, 2, 0.5, 17)
    assert o.steps_used[0] == 17 and t == 16
    assert o.out_tokens[0].tolist() == hist[16]


def test_mean_entropy_threshold_is_strict():
    t, o, _ = run([[1, 2, 3, 4]] * 40, 0.5, 2, 0.5, 10)       # mean == tau exactly -> never converges
    assert o.steps_used[0] == 10
    t, o, _ = run([[1, 2, 3, 4]] * 40, 0.4999, 2, 0.5, 10)
    assert o.steps_used[0] == 3


def test_one_change_resets_the_count():
    hist = [[1, 1, 1, 1]] * 3 + [[1, 1, 1, 2]] + [[1, 1, 1, 2]] * 10
    t, o, _ = run(hist, 0.0, 3, 0.5, 32)
    assert o.steps_used[0] == 7        # equalities at steps 1,2 then reset at 3, then 4,5,6


def test_denoise_case_accounting():
    st = fresh(1, 4)
    cv.converged(np.zeros((1, 4)), np.zeros((1, 4)), st, 2, 0.5, 32, [1], 10)
    o = cv.converged(np.array([[1, 2, 3, 4]]), np.ones((1, 4)), st, 2, 0.5, 32, [1], 10)
    assert o.num_sampled[0] == 0 and o.committed[0] == 0 and st.sc_on[0] == 1 and st.step_in_block[0] == 1
    assert st.prev_argmax[0].tolist() == [1, 2, 3, 4]
