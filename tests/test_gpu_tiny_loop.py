"""The tiny closed loop on the GPU (through the C ABI) against the oracle loop, free-running.

Trajectories must be identical until the first counted near-tie (argmax or Gumbel-key gap
< 1e-5, running entropy within 1e-3 of the budget, mean entropy within 1e-3 of tau, or
the last accepted and first rejected entropies within 1e-3); after one, divergence is reported.
"""
import numpy as np
import pytest

import synth
from oracle import loop as oloop
from synth.configs import TINY_LOOP
from tests import parity as P

pytestmark = pytest.mark.gpu


def _near_tie(o):
    """The tie class of step o, or None: argmax / Gumbel-key gaps, the running entropy at the
    budget, the mean entropy at tau, or the two entropies at the acceptance cut (the last accepted
    and the first rejected position in (entropy, position) order) within 1e-3."""
    if np.any((o["argmax_gap"] > 0) & (o["argmax_gap"] < P.TIE_GAP)):
        return "argmax_gap"
    if np.any(o["key_gap"] < P.TIE_GAP):
        return "gumbel_key_gap"
    if o["budget_gap"] < P.BUDGET_TIE:
        return "budget"
    if o["mean_gap"] < P.MEAN_TIE:
        return "mean_entropy"
    h = np.asarray(o["entropy"])
    order = np.lexsort((np.arange(h.size), h))
    n = o["n_accept"]
    if 0 < n < h.size and h[order[n]] - h[order[n - 1]] < 1e-3:
        return "accept_cut"
    return None


@pytest.mark.parametrize("scale", [4.0, 8.0, 32.0])
def test_tiny_loop_free_run(scale):
    from denoise_step_amd.tiny_loop import TinyLoop
    print(f"tiny loop scale={scale}", flush=True)
    inp = synth.tiny_loop_inputs(TINY_LOOP, None if scale == 4.0 else scale)
    ref = oloop.tiny_loop(TINY_LOOP, inp)
    got = TinyLoop(TINY_LOOP, inp).run(record=True)
    for t, (g, o) in enumerate(zip(got["traj"], ref["traj"])):
        assert np.abs(g["logits"] - o["logits"]).max() < 1e-3, t
        assert np.abs(g["entropy"] - o["entropy"]).max() < P.TOL_ENTROPY, t
        tie = _near_tie(o)
        same = (np.array_equal(g["argmax"], o["argmax"]) and np.array_equal(g["sample"], o["sample"])
                and g["n_accept"] == o["n_accept"] and np.array_equal(g["canvas"], o["canvas"])
                and g["committed"] == o["committed"])
        if not same:
            assert tie is not None, f"trajectories diverge at step {t} without a near-tie"
            P.report_tie(tie)
            P.report_tie("tiny_loop_divergence")
            return
        assert P.rel_norm_err(g["x_next"], o["x_next"]).max() < 1e-4, t
    assert got["steps_used"] == ref["steps_used"]
    assert np.array_equal(got["tokens"], ref["tokens"])
    assert np.abs(got["k_cache"] - ref["k_cache"]).max() < 1e-4
    if scale == 4.0:
        assert got["steps_used"] == TINY_LOOP["max_steps"]
    if scale == 32.0:
        assert got["steps_used"] == TINY_LOOP["k"] + 1
