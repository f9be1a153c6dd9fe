"""The tiny closed denoise loop: prefill, denoise steps until commit, commit pass.

Follows the DiffusionGemma/vLLM page, section "Two modes, one set of weights"
(the loop of one block: prompt prefill by the encoder, random canvas, denoise
steps with the decoder until the block stops changing, final encoder pass that
writes the block's K/V and emits its tokens) and section
"DiffusionGemmaModelState and DiffusionSampler" (prefill / denoise / commit
cases).  Each denoise step runs, in order: backbone (decoder) -> sampler ->
entropy-budget accept -> convergence -> self-conditioning for the next step.

Pinned by tests/test_oracle_traces.py: two constructed inputs with closed-form
dynamics (a one-hot case whose block converges after k + 1 steps with the
prefill canvas as its tokens and its commit pass appended after the prefix;
an equal-entropy case where the budget accepts exactly two positions per step,
the others are renoised from Philox RENOISE at the step's global step, and the
block runs to the cap and restarts from Philox INIT); tests/test_oracle_loop.py
checks determinism and the dynamics the workload's constants imply.
"""
from __future__ import annotations

import numpy as np

from . import accept as acc_mod
from . import backbone, converged as conv_mod, sampler, selfcond


def tiny_loop(cfg: dict, inp: dict, record: bool = True) -> dict:
    V, C, d = cfg["V"], cfg["C"], cfg["d"]
    Hq, Hkv, D, ps = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["page_size"]
    T = cfg["temperature"]
    E = np.asarray(inp["E"], np.float64)
    w = {k: np.asarray(inp[k], np.float64) for k in ("wq", "wk", "wv", "wo")}
    tbl = inp["page_table"]
    n_pages = int(inp["n_pages_total"])
    kc = np.zeros((n_pages, Hkv, ps, D))
    vc = np.zeros((n_pages, Hkv, ps, D))
    seeds = np.array([inp["seed64"]], np.uint64)
    P0 = cfg["prefix"]

    # encoder prefill: causal rows, K/V written
    x = E[np.asarray(inp["prefix"], np.int64)]
    _, kc, vc = backbone.layer(x, w, kc, vc, tbl, (0, 0, P0, 0, 0), Hq, Hkv, D, ps)

    state = conv_mod.LoopState(canvas=np.zeros((1, C), np.int64), prev_argmax=np.zeros((1, C), np.int64),
                               unchanged=np.zeros(1, np.int64), step_in_block=np.full(1, -1, np.int64),
                               step_global=np.zeros(1, np.int64), sc_on=np.zeros(1, np.uint8))
    conv_mod.converged(np.zeros((1, C), np.int64), np.zeros((1, C)), state, cfg["k"], cfg["tau"],
                       cfg["max_steps"], seeds, V)          # prefill case: random canvas
    traj = []
    x = E[state.canvas[0]]
    result = None
    for _t in range(cfg["max_steps"]):
        steps_now = state.step_global.copy()
        h, _, _ = backbone.layer(x, w, kc, vc, tbl, (0, P0, 0, C, 0), Hq, Hkv, D, ps)
        logits = backbone.lm_head(h, E, inp["logit_scale"])
        so = sampler.denoise_sample(logits, T, seeds, steps_now, C)
        ao = acc_mod.entropy_accept(so.entropy[None, :], so.sample[None, :], state.canvas, cfg["budget"],
                                    seeds, steps_now, V)
        state.canvas[:] = ao.canvas
        co = conv_mod.converged(so.argmax[None, :], so.entropy[None, :], state, cfg["k"], cfg["tau"],
                                cfg["max_steps"], seeds, V)
        P = selfcond.probs_from_stats(logits, T, so.row_max, so.row_lnz)
        x, _s, _y = selfcond.selfcond_embed(P, state.canvas, state.sc_on, E, inp["w_gate"], inp["w_up"],
                                            inp["w_down"], C, to_bf16=False)
        if record:
            traj.append(dict(logits=logits, entropy=so.entropy.copy(), argmax=so.argmax.copy(),
                             sample=so.sample.copy(), n_accept=int(ao.n_accept[0]),
                             canvas=state.canvas[0].copy(), committed=int(co.committed[0]),
                             argmax_gap=so.argmax_gap.copy(), key_gap=so.key_gap.copy(),
                             budget_gap=float(ao.budget_gap[0]), mean_gap=float(co.mean_gap[0]),
                             x_next=x.copy()))
        if co.committed[0]:
            result = dict(tokens=co.out_tokens[0].copy(), steps_used=int(co.steps_used[0]))
            break
    # encoder commit pass: the committed tokens' K/V are appended after the prefix
    xc = E[result["tokens"]]
    _, kc, vc = backbone.layer(xc, w, kc, vc, tbl, (0, P0, C, 0, 0), Hq, Hkv, D, ps)
    result.update(traj=traj, k_cache=kc, v_cache=vc)
    return result
