"""The tiny closed loop: determinism and the dynamics its constants imply (hand-worked traces: test_oracle_traces.py)."""
import numpy as np

import synth
from oracle import loop
from synth.configs import TINY_LOOP


def test_tiny_loop_deterministic_and_caps():
    inp = synth.tiny_loop_inputs(TINY_LOOP)
    a = loop.tiny_loop(TINY_LOOP, inp)
    b = loop.tiny_loop(TINY_LOOP, inp)
    assert np.array_equal(a["tokens"], b["tokens"]) and a["steps_used"] == b["steps_used"]
    # logit scale 4 keeps every position near-uniform (H ~ 6.6 nats > 2.0 budget): runs to the cap
    assert a["steps_used"] == TINY_LOOP["max_steps"]
    assert all(t["n_accept"] == 0 for t in a["traj"])


def test_tiny_loop_sharp_variant_converges_in_k_plus_1():
    inp = synth.tiny_loop_inputs(TINY_LOOP, variant_scale=32.0)
    r = loop.tiny_loop(TINY_LOOP, inp)
    assert r["steps_used"] == TINY_LOOP["k"] + 1
    assert np.mean(r["traj"][-1]["entropy"]) < TINY_LOOP["tau"]
    # the commit pass appended the block's K/V after the prefix
    assert r["k_cache"].shape[2] == TINY_LOOP["page_size"]
