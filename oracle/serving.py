"""The batched serving loop with deficit admission, composed from the oracle's pinned parts.

Test infrastructure (the oracle of denoise_step_amd.serving).  Per iteration, following the Sangam
page (section on the deficit token-budget scheduler) for admission and the DiffusionGemma/vLLM page
(sections "Two modes, one set of weights", "Dynamic per-sequence causal attention",
"Entropy-based denoising", "DiffusionGemmaModelState and DiffusionSampler") for the phases:
  1. requests arriving at this iteration join a first-come-first-served queue;
  2. decode work = C tokens for every request that denoises or runs a commit pass;
  3. admission.admit decides whether the queue head is prefilled, whole, in this iteration;
  4. one mixed attention launch over the scheduled requests in request order (prefill: the
     prompt as causal rows over an empty cache; denoise: C canvas rows over the cache; commit:
     C causal rows appended after the cache);
  5. denoising requests: sampler (logit pool entry it mod n_pool, request r's rows r*C ..), entropy
     accept, convergence; a request prefilled in this iteration gets its first canvas from the
     prefill case of the convergence step;
  6. transitions: prefill -> denoise; a committed block -> commit pass next iteration; after the
     commit pass of its last block a request is done.
With self-conditioning (DiffusionGemma/vLLM page, section "Self-conditioning"), each iteration with
denoising requests also forms the next step's canvas embedding of their rows from this iteration's
softmax, after the convergence step: x_next = E[canvas] + (sc_on ? MLP(P . E) : 0).
A steady-state start puts every request in the denoising phase over its cached prefix, with its
first canvas from the prefill case at global step g0 - 1 and the counters (step in block s0, global
step g0, self-conditioning on when s0 > 0).

Pinned by tests/test_oracle_traces.py against the hand-worked schedule of
tests/golden/serving_trace.txt (admissions, tokens and deficit per iteration, the split of every
launch, the commit iterations, the first canvases and where each causal pass's K/V land).
"""
from __future__ import annotations

import numpy as np

from . import accept as acc_mod
from . import admission, attention, converged as conv_mod, sampler, selfcond as sc_mod


def _bf16(a):
    a = np.asarray(a, np.uint16).astype(np.uint32) << 16
    return a.view(np.float32).astype(np.float64)


def serving_loop(cfg: dict, sched: dict, tensors: dict, max_iters: int = 10000, selfcond: dict | None = None,
                 start: dict | None = None) -> list:
    """Returns one record per iteration: admitted ids, tokens, deficit, launch splits, attention
    output [rows, Hq, D], commits {request: tokens}, canvas [R, C] after the iteration, and with
    selfcond (fp64 E [V, d], w_gate, w_up, w_down) x_next [R * C, d] (rows of denoising requests;
    NaN elsewhere).  start: dict(cached, step_in_block, step_global) per request."""
    R, C, V, ps = cfg["R"], cfg["C"], cfg["V"], cfg["page_size"]
    q, k, v = _bf16(tensors["q"]), _bf16(tensors["k"]), _bf16(tensors["v"])
    kc, vc = _bf16(tensors["k_cache"]), _bf16(tensors["v_cache"])
    logits = tensors["logits"]
    seeds = sched["seeds"]
    prompt, arrival, page0 = sched["prompt"], sched["arrival"], sched["page0"]
    tbl = sched["page_table"]
    state = conv_mod.LoopState(canvas=np.zeros((R, C), np.int64), prev_argmax=np.zeros((R, C), np.int64),
                               unchanged=np.zeros(R, np.int64), step_in_block=np.full(R, -1, np.int64),
                               step_global=np.zeros(R, np.int64), sc_on=np.zeros(R, np.uint8))
    phase = ["waiting"] * R
    cached = [0] * R
    blocks = [0] * R
    if start is not None:
        state.step_global[:] = np.asarray(start["step_global"], np.int64) - 1
        conv_mod.converged(np.zeros((R, C), np.int64), np.zeros((R, C)), state, cfg["k"], cfg["tau"],
                           cfg["max_steps"], seeds, V)                    # prefill case: first canvases
        state.step_in_block[:] = np.asarray(start["step_in_block"], np.int64)
        state.sc_on[:] = (state.step_in_block > 0).astype(np.uint8)
        phase = ["denoise"] * R
        cached = [int(c) for c in start["cached"]]
    queue, deficit = [], 0
    log = []
    for it in range(max_iters):
        if all(p == "done" for p in phase):
            break
        if start is None:                          # a steady-state start has admitted every request
            queue += [r for r in range(R) if arrival[r] == it]
        decode = C * sum(p in ("denoise", "commit") for p in phase)
        n, deficit, tokens = admission.admit(cfg["token_budget"], decode, [int(prompt[r]) for r in queue], deficit)
        admitted, queue = queue[:n], queue[n:]
        for r in admitted:
            phase[r] = "prefill"
        splits, row = [], 0
        for r in range(R):
            if phase[r] == "prefill":
                sp = (row, 0, int(prompt[r]), 0, int(page0[r]))
            elif phase[r] == "denoise":
                sp = (row, cached[r], 0, C, int(page0[r]))
            elif phase[r] == "commit":
                sp = (row, cached[r], C, 0, int(page0[r]))
            else:
                continue
            splits.append(sp)
            row += sp[2] + sp[3]
        out = None
        if row > 0:
            out, kc, vc = attention.canvas_attention(q[:row], k[:row], v[:row], kc, vc, tbl, splits, ps,
                                                     1.0 / np.sqrt(cfg["D"]))
        den = np.array([p == "denoise" for p in phase])
        act = np.array([p in ("denoise", "prefill") for p in phase])
        rec = dict(iteration=it, admitted=admitted, tokens=tokens, deficit=deficit, splits=splits,
                   attention=out, committed={}, gaps=[])
        argmax = np.zeros((R, C), np.int64)
        entropy = np.zeros((R, C))
        if den.any():
            steps_now = state.step_global.copy()
            so = sampler.denoise_sample(_bf16(logits[it % cfg["n_pool"]]), cfg["temperature"], seeds, steps_now, C,
                                        active=den)
            ao = acc_mod.entropy_accept(so.entropy.reshape(R, C), so.sample.reshape(R, C), state.canvas,
                                        cfg["budget"], seeds, steps_now, V, active=den)
            state.canvas[den] = ao.canvas[den]
            argmax, entropy = so.argmax.reshape(R, C), so.entropy.reshape(R, C)
            rec["gaps"] = [so.argmax_gap, so.key_gap, ao.budget_gap]
        co = None
        if act.any():
            co = conv_mod.converged(argmax, entropy, state, cfg["k"], cfg["tau"], cfg["max_steps"], seeds, V,
                                    active=act)
            rec["mean_gap"] = co.mean_gap
        rec["canvas"] = state.canvas.copy()
        if selfcond is not None and den.any():
            P = sc_mod.probs_from_stats(_bf16(logits[it % cfg["n_pool"]]), cfg["temperature"], so.row_max, so.row_lnz)
            x, _s, _y = sc_mod.selfcond_embed(P, state.canvas, state.sc_on, selfcond["E"], selfcond["w_gate"],
                                              selfcond["w_up"], selfcond["w_down"], C, to_bf16=False)
            x[~np.repeat(den, C)] = np.nan
            rec["x_next"] = x
        for r in range(R):
            if phase[r] == "prefill":
                cached[r] = int(prompt[r])
                phase[r] = "denoise"
            elif phase[r] == "commit":
                cached[r] += C
                phase[r] = "denoise" if blocks[r] < cfg["blocks"] else "done"
            elif phase[r] == "denoise" and co is not None and co.committed[r]:
                rec["committed"][r] = co.out_tokens[r].copy()
                blocks[r] += 1
                phase[r] = "commit"
        log.append(rec)
    rec_final = dict(k_cache=kc, v_cache=vc)
    return log, rec_final
