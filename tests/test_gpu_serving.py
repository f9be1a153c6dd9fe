"""The serving loop on the GPU (through the C ABI) against oracle.serving and the oracle's parts.

Small configuration, whole loop: every iteration must agree exactly in its schedule (admitted
prefill, tokens, deficit, launch splits), its attention output within the bf16 tolerance, its
canvases, commits and next-step embeddings x_next (self-conditioning on), until the first counted
near-tie (argmax or Gumbel-key gap < 1e-5, running entropy within 1e-3 of the budget, mean entropy
within 1e-3 of tau); after one, divergence is reported.  The final paged caches (prompt,
commit-pass appends and untouched pages) must be identical.

Batched workload at its stated size (32 requests, prefixes U[512, 8192], 256-token canvases at
staggered steps, V = 262144, d = 4096): the loop runs long enough for three blocks to hit the step
cap, commit, run their commit pass and restart; two requests are checked in lockstep against the
oracle's parts from the GPU's own state before each iteration.
"""
import numpy as np
import pytest

import synth
from oracle import accept as oacc
from oracle import attention as oatt
from oracle import converged as oconv
from oracle import sampler as osamp
from oracle import selfcond as osc
from oracle import serving as oserving
from synth import configs
from synth.configs import SERVING_SMALL
from tests import parity as P

pytestmark = pytest.mark.gpu


def _tie(o):
    if not o["gaps"]:
        return False
    ag, kg, bg = o["gaps"]
    if np.any((ag > 0) & (ag < P.TIE_GAP)) or np.any(kg < P.TIE_GAP) or np.any(bg < P.BUDGET_TIE):
        return True
    return bool(np.any(o.get("mean_gap", np.inf) < P.MEAN_TIE))


@pytest.mark.parametrize("budget", [72, 40])
def test_serving_loop_matches_oracle(budget):
    import torch

    import denoise_step_amd as dg
    from denoise_step_amd.serving import ServingLoop
    cfg = dict(SERVING_SMALL, token_budget=budget)
    print(f"serving loop small, token budget {budget}, self-conditioning on", flush=True)
    sched = synth.serving_schedule_inputs(cfg)
    host = synth.serving_small_tensors(cfg, sched)
    V, d, h = cfg["V"], cfg["d"], cfg["hidden"]
    E = synth.normal_bf16(cfg["seed"], "serving.E", (V, d), 1 / 8)
    w = [synth.normal_bf16(cfg["seed"], t, sh, 0.5) for t, sh in (("serving.wg", (d, h)), ("serving.wu", (d, h)),
                                                                  ("serving.wd", (h, d)))]
    f = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64)
    ref, fin = oserving.serving_loop(cfg, sched, host, selfcond=dict(E=f(E), w_gate=f(w[0]), w_up=f(w[1]),
                                                                     w_down=f(w[2])))
    dev = {k: P.dev_bf16(v) for k, v in host.items()}
    Et = P.dev_bf16(E)
    prepared = dg.dg_selfcond_prepare(Et, *(P.dev_bf16(a) for a in w))
    got = ServingLoop(cfg, sched, dev, selfcond=dict(E=Et, prepared=prepared, hidden=h)).run(record=True)
    assert len(got) >= 1
    tied = False
    n_x = 0
    for g, o in zip(got, ref):
        t = g["iteration"]
        assert (g["admitted"], g["tokens"], g["deficit"]) == (o["admitted"], o["tokens"], o["deficit"]), t
        assert g["splits"][:, :5].tolist() == [list(s) for s in o["splits"]], t
        err = np.abs(g["attention"] - o["attention"]).max()
        assert err <= P.TOL_ATT_BF16, (t, err)
        tied = tied or _tie(o)
        same = np.array_equal(g["canvas"], o["canvas"]) and sorted(g["committed"]) == sorted(o["committed"]) and all(
            np.array_equal(g["committed"][r], o["committed"][r]) for r in g["committed"])
        if not same:
            assert tied, f"serving loop diverges at iteration {t} without a near-tie"
            P.report_tie("serving_divergence")
            return
        if "x_next" in o:
            rows = ~np.isnan(o["x_next"][:, 0])
            P.check_bf16_output(g["x_next"][rows], o["x_next"][rows])
            n_x += 1
    assert len(got) == len(ref) and n_x > 0
    torch.cuda.synchronize()
    assert np.array_equal(P.host_f64(dev["k_cache"]), fin["k_cache"])
    assert np.array_equal(P.host_f64(dev["v_cache"]), fin["v_cache"])


def test_batched_loop_lockstep_sampled_requests():
    """32 requests at staggered steps (request r at step 2r of its 64-step block), 7 iterations with
    self-conditioning: requests 31, 30 and 29 hit the cap at iterations 1, 3 and 5, commit their
    argmax, run the 256-row commit pass the next iteration and restart from a fresh Philox canvas
    with self-conditioning off.  Requests 31 and 0 are checked every iteration against the oracle's
    parts from the GPU's own state: every attention row (and the appended pages of a commit pass),
    the sampler outputs of 32 rows each (first, last and 30 random positions), accept and converged
    on the whole canvas exactly (fed the GPU's sampler outputs), and x_next of 4 rows each (fp64 P.E
    over table slabs)."""
    torch = P.torch_mod()
    import denoise_step_amd as dg
    from denoise_step_amd.serving import COMMIT, DENOISE, ServingLoop
    cfg = configs.BATCHED_LOOP
    R, C, V, d, h = cfg["R"], cfg["C"], cfg["V"], cfg["d"], cfg["hidden"]
    Hq, Hkv, D, ps = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["page_size"]
    print("batched loop: 32 x 256 canvases, V = 262144, d = 4096, self-conditioning", flush=True)
    sched = synth.serving_schedule_inputs(cfg)
    start = synth.batched_loop_start(cfg, sched)
    n = R * C
    bf = torch.bfloat16
    g = lambda tag, shape, std=1.0: synth.normal_torch(cfg["seed"], ("bloop", tag), shape, std, bf, "cuda")
    t = dict(q=g("q", (n, Hq, D)), k=g("k", (n, Hkv, D)), v=g("v", (n, Hkv, D)),
             k_cache=g("kc", (sched["n_pages"], Hkv, ps, D)), v_cache=g("vc", (sched["n_pages"], Hkv, ps, D)))
    t["logits"] = torch.empty((cfg["n_pool"], n, V), dtype=bf, device="cuda")
    for i in range(cfg["n_pool"]):
        t["logits"][i] = synth.zipf_logits_torch(cfg["seed"], ("bloop.logits", i), n, V, "cuda")
    E = g("E", (V, d), 1 / 8)
    w = [g(tag, sh, 0.02) for tag, sh in (("wg", (d, h)), ("wu", (d, h)), ("wd", (h, d)))]
    prepared = dg.dg_selfcond_prepare(E, *w)
    f = lambda x: x.float().cpu().numpy().astype(np.float64)
    wh = [f(x) for x in w]
    loop = ServingLoop(cfg, sched, t, selfcond=dict(E=E, prepared=prepared, hidden=h), start=start)
    seeds = sched["seeds"]
    watch = (31, 0)
    commits = {}
    pending = []
    for it in range(7):
        print(f"  iteration {it}", flush=True)
        sp, rows = loop._splits()
        before = {}
        for r in watch:
            i = [k for k in range(sp.shape[0]) if sp[k, 4] == sched["page0"][r]][0]
            p0 = int(sched["page0"][r])
            p1 = int(sched["page0"][r + 1]) if r + 1 < R else sched["page_table"].size
            pages = sched["page_table"][p0:p1].astype(np.int64)
            pt = torch.as_tensor(pages, device="cuda")
            st = {k: v[r].cpu().numpy().copy() for k, v in loop.state.items()}
            before[r] = dict(split=sp[i].copy(), phase=loop.phase[r], kc=f(t["k_cache"][pt]), vc=f(t["v_cache"][pt]),
                             pages=pt, state=st)
        rec = loop.step(it)
        commits[it] = sorted(rec["committed"])
        torch.cuda.synchronize()
        logits = t["logits"][it % cfg["n_pool"]]
        for r in watch:
            b = before[r]
            row0, cached, nc, nv = (int(x) for x in b["split"][:4])
            nr = nc + nv
            sl = slice(row0, row0 + nr)
            # attention: every row, the request alone over its own pages
            kc, vc = b["kc"], b["vc"]
            local = np.arange(kc.shape[0], dtype=np.int32)
            out, kc2, vc2 = oatt.canvas_attention(f(t["q"][sl]), f(t["k"][sl]), f(t["v"][sl]), kc, vc, local,
                                                  [(0, cached, nc, nv, 0)], ps, 1.0 / np.sqrt(D))
            err = np.abs(f(loop.last["attention"][sl]) - out).max()
            assert err <= P.TOL_ATT_BF16, (it, r, err)
            if nc:
                assert np.array_equal(f(t["k_cache"][b["pages"]]), kc2) and np.array_equal(f(t["v_cache"][b["pages"]]),
                                                                                          vc2), (it, r)
            if b["phase"] != DENOISE:
                assert b["phase"] == COMMIT
                continue
            # sampler on this request's rows (its seed and global step)
            rows_r = np.arange(r * C, (r + 1) * C)
            check = rows_r[np.unique(np.r_[0, C - 1, synth.rng_for(it, r, "bloop.rows").choice(C, 30, replace=False)])]
            host_l = f(logits[torch.as_tensor(check, device="cuda")])
            so_ref = osamp.SampleOut(*(np.zeros(n) for _ in range(5)), argmax_gap=np.zeros(n), key_gap=np.zeros(n))
            for j, row in enumerate(check):
                one = P.sampler_oracle_row(host_l[j], int(seeds[r]), int(row - r * C), int(b["state"]["step_global"]))
                for fld in ("entropy", "argmax", "sample", "row_max", "row_lnz", "argmax_gap", "key_gap"):
                    getattr(so_ref, fld)[row] = getattr(one, fld)[0]
            got_so = {k: v.cpu().numpy()[check] for k, v in loop.so.items()}
            P.check_sampler_rows(got_so, so_ref, list(check))
            # accept and converged from the GPU's sampler outputs and the pre-step state
            H = loop.so["entropy"].cpu().numpy()[rows_r][None, :].astype(np.float64)
            samp = loop.so["sample"].cpu().numpy()[rows_r][None, :]
            am = loop.so["argmax"].cpu().numpy()[rows_r][None, :]
            s0 = b["state"]
            ost = oconv.LoopState(canvas=s0["canvas"][None, :].astype(np.int64),
                                  prev_argmax=s0["prev_argmax"][None, :].astype(np.int64),
                                  unchanged=np.array([s0["unchanged"]], np.int64),
                                  step_in_block=np.array([s0["step_in_block"]], np.int64),
                                  step_global=np.array([s0["step_global"]], np.int64),
                                  sc_on=np.array([s0["sc_on"]], np.uint8))
            ao = oacc.entropy_accept(H, samp, ost.canvas, cfg["budget"], [int(seeds[r])], ost.step_global, V)
            tie = ao.budget_gap[0] < P.BUDGET_TIE
            ost.canvas[:] = ao.canvas
            co = oconv.converged(am, H, ost, cfg["k"], cfg["tau"], cfg["max_steps"], [int(seeds[r])], V)
            got_st = {k: v[r].cpu().numpy() for k, v in loop.state.items()}
            if tie and not np.array_equal(got_st["canvas"], ost.canvas[0]):
                P.report_tie("budget")
                continue
            for fld in ("canvas", "prev_argmax", "unchanged", "step_in_block", "step_global", "sc_on"):
                assert np.array_equal(np.asarray(got_st[fld]).astype(np.int64),
                                      getattr(ost, fld)[0].astype(np.int64)), (it, r, fld)
            assert bool(r in rec["committed"]) == bool(co.committed[0]), (it, r)
            if co.committed[0]:
                assert np.array_equal(rec["committed"][r], co.out_tokens[0]), (it, r)
            # x_next of 4 rows: E[canvas'] + (sc_on' ? MLP(P . E) : 0), checked after the loop
            sel = rows_r[[0, 77, 200, 255]]
            hl = f(logits[torch.as_tensor(sel, device="cuda")])
            ref4 = osamp.denoise_sample(hl, 1.0, [int(seeds[r])], [int(s0["step_global"])], 4)
            tok = torch.as_tensor(ost.canvas[0][sel - r * C].astype(np.int64), device="cuda")
            pending.append(dict(P=osc.probs_from_stats(hl, 1.0, ref4.row_max, ref4.row_lnz), e=f(E[tok]),
                                on=bool(ost.sc_on[0]), x=f(loop.x[torch.as_tensor(sel, device="cuda")]), it=it))
    # three blocks reached the cap on schedule, each followed by its commit pass
    assert commits[1] == [31] and commits[3] == [30] and commits[5] == [29], commits
    # one pass of fp64 P.E over the table for every collected row
    s_ref = P.oracle_pe_slabs(np.concatenate([c["P"] for c in pending]), P.torch_table_rows(E), V)
    y_ref = osc.gated_mlp(s_ref, *wh)
    for i, c in enumerate(pending):
        P.check_bf16_output(c["x"], c["e"] + (y_ref[4 * i:4 * i + 4] if c["on"] else 0.0))
    assert any(not c["on"] for c in pending) and any(c["on"] for c in pending)


def test_serving_loop_checkpoint_resume():
    """Checkpoint / resume: a loop that runs some iterations, is checkpointed and continues, against a
    fresh loop (its own workspaces, KV cache and state buffers) restored from that checkpoint and run
    over the same iterations: schedules, attention outputs, canvases, commits, next-step embeddings
    and the final state and caches must be bitwise equal."""
    import torch

    import denoise_step_amd as dg
    from denoise_step_amd.serving import DONE, ServingLoop
    cfg = dict(SERVING_SMALL, token_budget=72)
    print("serving loop small: checkpoint after 6 iterations, resume in a fresh loop", flush=True)
    sched = synth.serving_schedule_inputs(cfg)
    host = synth.serving_small_tensors(cfg, sched)
    V, d, h = cfg["V"], cfg["d"], cfg["hidden"]
    E = P.dev_bf16(synth.normal_bf16(cfg["seed"], "serving.E", (V, d), 1 / 8))
    w = [P.dev_bf16(synth.normal_bf16(cfg["seed"], t, sh, 0.5))
         for t, sh in (("serving.wg", (d, h)), ("serving.wu", (d, h)), ("serving.wd", (h, d)))]
    prepared = dg.dg_selfcond_prepare(E, *w)
    sc = dict(E=E, prepared=prepared, hidden=h)

    def fresh():
        return ServingLoop(cfg, sched, {k: P.dev_bf16(v) for k, v in host.items()}, selfcond=sc)

    first = 6
    a = fresh()
    for it in range(first):
        a.step(it)
    ck = a.checkpoint()
    b = fresh()
    b.restore(ck)
    recs = {}
    for name, loop in (("continued", a), ("resumed", b)):
        out = []
        for it in range(first, first + 40):
            if np.all(loop.phase == DONE):
                break
            r = loop.step(it, record=True)
            r.pop("gpu_ms")
            out.append(r)
        torch.cuda.synchronize()
        recs[name] = out
    assert len(recs["continued"]) == len(recs["resumed"]) > 5
    n_commit = 0
    for g, o in zip(recs["continued"], recs["resumed"]):
        t = g["iteration"]
        assert (g["admitted"], g["tokens"], g["deficit"]) == (o["admitted"], o["tokens"], o["deficit"]), t
        assert ("splits" in g) == ("splits" in o), t
        if "splits" in g:
            assert np.array_equal(g["splits"], o["splits"]), t
        if "attention" in g:
            assert np.array_equal(g["attention"], o["attention"]), t
        assert np.array_equal(g["canvas"], o["canvas"]), t
        assert sorted(g["committed"]) == sorted(o["committed"]), t
        assert all(np.array_equal(g["committed"][r], o["committed"][r]) for r in g["committed"]), t
        n_commit += len(g["committed"])
        if "x_next" in g:
            assert np.array_equal(g["x_next"], o["x_next"]), t
    assert n_commit >= 1
    for k in a.state:
        assert torch.equal(a.state[k], b.state[k]), k
    assert torch.equal(a.t["k_cache"], b.t["k_cache"]) and torch.equal(a.t["v_cache"], b.t["v_cache"])
