"""Hand-worked traces that pin the oracle's compositions: the one-layer backbone, the tiny closed
loop and the serving loop (the pages print no trajectory, so the expected values are derived by
hand from the pages' rules, or follow from closed forms, never from running the oracle).

Backbone and serving: tests/golden/backbone_trace.txt and tests/golden/serving_trace.txt (each
with its derivation and citations).  Loop: two constructed inputs whose dynamics have closed forms
(DiffusionGemma/vLLM page, sections "Entropy-based denoising", "Two modes, one set of weights" and
"DiffusionGemmaModelState and DiffusionSampler"):
  * sharp: one-hot embeddings and a logit gap of 40 (> 20.2, the widest spread of two Gumbel
    values the noise mapping can produce), zero attention output and MLP, so the sample is the
    argmax, every position is accepted, the canvas never changes and the block converges after
    k + 1 steps with the initial (prefill) canvas as its tokens;
  * budget: V = 2 with logits 2 * onehot(canvas), so every position has the same entropy
    H = ln(1 + e^-2) + 2 e^-2 / (1 + e^-2) = 0.36533 nats; a budget of 1.0 accepts exactly the
    positions 0 and 1 (ties go to the lower position; 2 H <= 1 < 3 H), positions 2 and 3 are
    renoised every step, and tau = 0.3 < H keeps the block running to the cap.
"""
import math
import os

import numpy as np
import pytest

from oracle import backbone, loop, philox, serving

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_values(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, rest = line.split(None, 1)
            vals[key] = np.array([[float(t) for t in r.split()] for r in rest.split(";")])
    return vals


# ---------------------------------------------------------------- backbone
E4 = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [2.0, -1.0]])


def _layer(x, w, kc, vc, split):
    return backbone.layer(x, w, kc, vc, np.array([0]), split, 1, 1, 2, 16)


def test_backbone_uniform_trace():
    g = _golden_values("backbone_trace.txt")
    I, Z = np.eye(2), np.zeros((2, 2))
    w = dict(wq=Z, wk=Z, wv=I, wo=I)
    kc = np.zeros((1, 1, 16, 2))
    vc = np.zeros((1, 1, 16, 2))
    h, kc, vc = _layer(E4[[0, 1]], w, kc, vc, (0, 0, 2, 0, 0))            # encoder prefill
    np.testing.assert_allclose(h, g["uniform.prefill.h"], atol=1e-14)
    h, kc2, vc2 = _layer(E4[[2, 3]], w, kc, vc, (0, 2, 0, 2, 0))          # decoder pass over the canvas
    np.testing.assert_allclose(h, g["uniform.canvas.h"], atol=1e-14)
    np.testing.assert_allclose(backbone.lm_head(h, E4, 4.0), g["uniform.canvas.logits"], atol=1e-13)
    assert np.array_equal(vc2, vc) and np.array_equal(kc2, kc)             # canvas K/V never written
    h, kc, vc = _layer(E4[[2, 3]], w, kc, vc, (0, 2, 2, 0, 0))            # encoder commit pass
    np.testing.assert_allclose(h, g["uniform.commit.h"], atol=1e-14)
    np.testing.assert_allclose(vc[0, 0, :4], g["uniform.v_cache"], atol=0)
    assert not np.any(kc)


def test_backbone_scored_trace():
    g = _golden_values("backbone_trace.txt")
    c = math.sqrt(math.sqrt(2.0) * math.log(3.0))
    w = dict(wq=c * np.eye(2), wk=c * np.eye(2), wv=np.array([[1.0, 1.0], [0.0, 1.0]]),
             wo=np.array([[0.0, 1.0], [0.0, 0.0]]))
    kc = np.zeros((1, 1, 16, 2))
    vc = np.zeros((1, 1, 16, 2))
    h, kc, vc = _layer(E4[[0, 1]], w, kc, vc, (0, 0, 2, 0, 0))
    np.testing.assert_allclose(h, g["scored.prefill.h"], atol=1e-14)
    np.testing.assert_allclose(vc[0, 0, :2], g["scored.v_cache"], atol=0)
    np.testing.assert_allclose(kc[0, 0, :2], c * np.eye(2), atol=1e-15)


# ---------------------------------------------------------------- tiny loop
def _loop_case(V, C, a, scale, budget, k, tau, max_steps, prefix=(0, 1)):
    d = V
    cfg = dict(V=V, C=C, d=d, Hq=1, Hkv=1, D=d, page_size=16, temperature=1.0, prefix=len(prefix),
               budget=budget, k=k, tau=tau, max_steps=max_steps)
    Z = np.zeros((d, d))
    inp = dict(E=a * np.eye(V), wq=Z, wk=Z, wv=np.eye(d), wo=Z, w_gate=np.zeros((d, 4)), w_up=np.zeros((d, 4)),
               w_down=np.zeros((4, d)), prefix=np.array(prefix), page_table=np.array([1]), n_pages_total=2,
               logit_scale=scale, seed64=np.uint64(1234))
    return cfg, inp


def test_loop_sharp_trace_converges_after_k_plus_1_with_prefill_canvas():
    cfg, inp = _loop_case(V=4, C=4, a=2.0, scale=10.0, budget=2.0, k=2, tau=0.5, max_steps=32)
    r = loop.tiny_loop(cfg, inp)
    init = philox.random_tokens(1234, 0, np.arange(4), 4, philox.INIT)     # prefill case, global step 0
    assert r["steps_used"] == cfg["k"] + 1
    assert np.array_equal(r["tokens"], init)
    for t in r["traj"]:
        assert t["n_accept"] == 4 and np.array_equal(t["argmax"], init) and np.array_equal(t["sample"], init)
        np.testing.assert_array_equal(t["logits"], 40.0 * np.eye(4)[init])
        assert np.all(t["entropy"] < 1e-14)
    assert [t["committed"] for t in r["traj"]] == [0, 0, 1]
    # the canvas stays the prefill canvas until the commit, which restarts it from Philox INIT at the
    # committing step's global step (prefill at 0, denoise steps at 1, 2, 3)
    assert all(np.array_equal(t["canvas"], init) for t in r["traj"][:-1])
    assert np.array_equal(r["traj"][-1]["canvas"], philox.random_tokens(1234, 3, np.arange(4), 4, philox.INIT))
    # encoder passes wrote v = x: the prefix at positions 0, 1, the committed block at 2 .. 5
    np.testing.assert_array_equal(r["v_cache"][1, 0, :6], 2.0 * np.eye(4)[[0, 1, *init]])
    assert not np.any(r["k_cache"])


def test_loop_budget_trace_accepts_two_and_runs_to_the_cap():
    cfg, inp = _loop_case(V=2, C=4, a=1.0, scale=2.0, budget=1.0, k=2, tau=0.3, max_steps=5)
    r = loop.tiny_loop(cfg, inp)
    H = math.log1p(math.exp(-2.0)) + 2.0 * math.exp(-2.0) / (1.0 + math.exp(-2.0))
    assert H == pytest.approx(0.365334, abs=1e-6)
    assert r["steps_used"] == 5 and len(r["traj"]) == 5
    canvas = philox.random_tokens(1234, 0, np.arange(4), 2, philox.INIT)
    for t, rec in enumerate(r["traj"]):
        assert np.array_equal(rec["argmax"], canvas)                        # argmax of 2 onehot(canvas)
        np.testing.assert_allclose(rec["entropy"], H, atol=1e-15)
        assert rec["n_accept"] == 2
        if t == 4:                     # the cap commits and restarts the canvas (global step 5)
            assert np.array_equal(rec["canvas"], philox.random_tokens(1234, 5, np.arange(4), 2, philox.INIT))
            break
        renoise = philox.random_tokens(1234, 1 + t, np.arange(4), 2, philox.RENOISE)   # global step 1 + t
        assert np.array_equal(rec["canvas"][2:], renoise[2:])
        assert np.array_equal(rec["canvas"][:2], rec["sample"][:2])
        canvas = rec["canvas"]
    assert np.array_equal(r["tokens"], r["traj"][-1]["argmax"])
    assert [rec["committed"] for rec in r["traj"]] == [0, 0, 0, 0, 1]


# ---------------------------------------------------------------- serving loop
def _serving_golden():
    rows = []
    with open(os.path.join(GOLDEN, "serving_trace.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            it, adm, tok, dfc, spl, com = (c.strip() for c in line.split("|"))
            splits = {}
            for item in spl.split():
                r, vals = item.split(":")
                splits[int(r)] = tuple(int(v) for v in vals.split(","))
            rows.append(dict(it=int(it), admitted=[] if adm == "-" else [int(adm)], tokens=int(tok),
                             deficit=int(dfc), splits=splits, commits=[] if com == "-" else [int(com)]))
    return rows


def test_serving_trace_matches_hand_schedule():
    cfg = dict(R=3, C=4, V=64, page_size=16, Hq=2, Hkv=1, D=8, token_budget=8, blocks=1, budget=4.0, k=2,
               tau=0.0, max_steps=2, temperature=1.0, n_pool=2)
    page0 = np.array([0, 1, 2], np.int32)
    sched = dict(prompt=np.array([6, 10, 3]), arrival=np.array([0, 0, 1]), page0=page0,
                 page_table=np.array([2, 0, 1], np.int32), seeds=np.array([11, 12, 13], np.uint64))
    rng = np.random.default_rng(5)
    bf = lambda shape: (rng.normal(0, 1, shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    n = 16
    tensors = dict(q=bf((n, 2, 8)), k=bf((n, 1, 8)), v=bf((n, 1, 8)), k_cache=np.zeros((3, 1, 16, 8), np.uint16),
                   v_cache=np.zeros((3, 1, 16, 8), np.uint16), logits=bf((2, 3 * 4, 64)))
    log, final = serving.serving_loop(cfg, sched, tensors)
    want = _serving_golden()
    assert len(log) == len(want)
    for rec, w in zip(log, want):
        assert rec["iteration"] == w["it"]
        assert rec["admitted"] == w["admitted"] and rec["tokens"] == w["tokens"] and rec["deficit"] == w["deficit"]
        got = {[r for r in range(3) if page0[r] == s[4]][0]: tuple(s[:4]) for s in rec["splits"]}
        assert got == w["splits"], (w["it"], got)
        assert sorted(rec["committed"]) == w["commits"]
    # the prefill case drew each request's first canvas at its global step 0
    first = {0: 0, 1: 3, 2: 4}
    for r, it in first.items():
        init = philox.random_tokens(int(sched["seeds"][r]), 0, np.arange(4), 64, philox.INIT)
        assert np.array_equal(log[it]["canvas"][r], init)
    # K/V rows of each causal pass land at its positions: launch rows are the first rows of the pools
    kf = (tensors["k"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    kc = final["k_cache"]
    np.testing.assert_array_equal(kc[2, 0, :6], kf[0:6, 0])      # request 0 prefill (it 0, rows 0..5)
    np.testing.assert_array_equal(kc[2, 0, 6:10], kf[0:4, 0])    # its commit pass (it 3, rows 0..3)
    np.testing.assert_array_equal(kc[0, 0, :10], kf[4:14, 0])    # request 1 prefill (it 3, rows 4..13)
    np.testing.assert_array_equal(kc[0, 0, 10:14], kf[0:4, 0])   # its commit pass (it 6, rows 0..3)
    np.testing.assert_array_equal(kc[1, 0, :3], kf[4:7, 0])      # request 2 prefill (it 4, rows 4..6)
    np.testing.assert_array_equal(kc[1, 0, 3:7], kf[0:4, 0])     # its commit pass (it 7, rows 0..3)


def test_serving_steady_start_hand_schedule():
    """A steady-state start (every request already holds its prefix and denoises from the first
    iteration, at its own step): two requests, C = 4, prefixes 5 and 9, steps in block 0 and 3 of
    a 4-step block, global steps 1 and 7.  Worked out by hand: request 1 is at its last step, so it
    commits in iteration 0, runs its commit pass (4 causal rows after its 9 cached) in iteration 1
    and denoises again from iteration 2 over 13 cached tokens; request 0 commits in iteration 3.
    The first canvases are the prefill case's Philox INIT tokens at global steps 0 and 6; arrivals
    are ignored; with self-conditioning off for request 0 (step 0) and on for request 1 (step 3)."""
    cfg = dict(R=2, C=4, V=64, page_size=16, Hq=2, Hkv=1, D=8, token_budget=8, blocks=2, budget=4.0, k=2,
               tau=0.0, max_steps=4, temperature=1.0, n_pool=1)
    sched = dict(prompt=np.array([5, 9]), arrival=np.array([0, 0]), page0=np.array([0, 1], np.int32),
                 page_table=np.array([1, 0], np.int32), seeds=np.array([21, 22], np.uint64))
    rng = np.random.default_rng(9)
    bf = lambda shape: (rng.normal(0, 1, shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    tensors = dict(q=bf((8, 2, 8)), k=bf((8, 1, 8)), v=bf((8, 1, 8)), k_cache=bf((2, 1, 16, 8)),
                   v_cache=bf((2, 1, 16, 8)), logits=bf((1, 8, 64)))
    start = dict(cached=[5, 9], step_in_block=[0, 3], step_global=[1, 7])
    log, _ = serving.serving_loop(cfg, sched, tensors, max_iters=5, start=start)
    split = lambda rec: [tuple(int(v) for v in s[:4]) for s in rec["splits"]]
    assert split(log[0]) == [(0, 5, 0, 4), (4, 9, 0, 4)]
    assert sorted(log[0]["committed"]) == [1]
    assert split(log[1]) == [(0, 5, 0, 4), (4, 9, 4, 0)]
    assert split(log[2]) == [(0, 5, 0, 4), (4, 13, 0, 4)]
    assert sorted(log[3]["committed"]) == [0]
    assert split(log[4]) == [(0, 5, 4, 0), (4, 13, 0, 4)]
    assert all(rec["admitted"] == [] for rec in log)
    # request 1's block committed the canvas it was sampling; its restart canvas is INIT at global step 7
    assert np.array_equal(log[0]["canvas"][1], philox.random_tokens(22, 7, np.arange(4), 64, philox.INIT))
