"""GPU parity at the full sizes of the batched, structured-read and block-draft workloads.

Every launch runs at full size through the C ABI, with inputs generated on the GPU by the
shared seeded generators.  The oracle then checks: every row of the attention of the snapshotted
requests (its own append / gather / mask / dense-attention steps, per request), 8 logit rows of
every active request for the sampler (its first, last and 6 random positions), whole canvases for
accept and converged, 2 rows of every request for P.E and the MLP.
The K/V pages that causal rows append are compared bit-exactly for the sampled requests.
"""
import numpy as np
import pytest

import synth
from oracle import accept as oacc
from oracle import attention as oatt
from oracle import converged as oconv
from oracle import sampler as osamp
from oracle import selfcond as osc
from synth import configs
from tests import parity as P

pytestmark = pytest.mark.gpu


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _i64(a):
    return np.asarray(a, np.uint64).view(np.int64)


class AttLaunch:
    """One full-size paged attention launch (bf16) with inputs generated on the GPU."""

    def __init__(self, lay: synth.PagedLayout, Hq, Hkv, D, seed, tag):
        torch = P.torch_mod()
        bf = torch.bfloat16
        self.lay, self.Hq, self.Hkv, self.D = lay, Hq, Hkv, D
        ps = lay.page_size
        g = lambda name, shape: synth.normal_torch(seed, (tag, name), shape, 1.0, bf, "cuda")
        self.q = g("q", (lay.rows, Hq, D))
        self.k = g("k", (lay.rows, Hkv, D))
        self.v = g("v", (lay.rows, Hkv, D))
        self.kc = g("kc", (lay.n_pages, Hkv, ps, D))
        self.vc = g("vc", (lay.n_pages, Hkv, ps, D))
        self.pt = P.dev(lay.page_table)
        self.sp = P.dev(lay.split_array())
        self.max_rows = max(s.n_causal + s.n_canvas for s in lay.splits)
        self.max_keys = max(s.cached + s.n_causal + s.n_canvas for s in lay.splits)
        self.scale = 1.0 / np.sqrt(D)

    def snapshot(self, reqs):
        """Host fp64 copies of the listed requests' rows and pages, taken before the launch."""
        torch = P.torch_mod()
        snap = {}
        for i in reqs:
            s = self.lay.splits[i]
            r0, nr = int(self.lay.row0[i]), s.n_causal + s.n_canvas
            pages = torch.as_tensor(self.lay.pages_of(i).astype(np.int64), device="cuda")
            snap[i] = dict(q=_f64(self.q[r0:r0 + nr]), k=_f64(self.k[r0:r0 + nr]), v=_f64(self.v[r0:r0 + nr]),
                           kc=_f64(self.kc[pages]), vc=_f64(self.vc[pages]), pages=pages)
        return snap

    def run(self):
        import denoise_step_amd as dg
        return dg.dg_canvas_attention(self.q, self.k, self.v, self.kc, self.vc, self.pt, self.sp, self.max_rows,
                                      self.max_keys, self.scale)

    def check_all(self, out, reqs, snap):
        """Every row of each listed request against the oracle, one request at a time: requests that
        append causal rows from their snapshot (taken before the launch, `snap`), the others from their
        pages as the launch left them (it writes no page of theirs; page lists are disjoint)."""
        worst = 0.0
        for n, i in enumerate(reqs):
            h = snap[i] if i in snap else self.snapshot([i])[i]
            worst = max(worst, self.check(out, {i: h}))
            if n % 16 == 15:
                print(f"  {n + 1} requests checked", flush=True)
        return worst

    def check(self, out, snap):
        """Every row of every snapshotted request against the oracle; appended pages exactly."""
        torch = P.torch_mod()
        G = self.Hq // self.Hkv
        ps = self.lay.page_size
        worst = 0.0
        for i, h in snap.items():
            s = self.lay.splits[i]
            nr = s.n_causal + s.n_canvas
            local = np.arange(h["kc"].shape[0], dtype=np.int32)   # the request's pages, renumbered
            kc, vc = h["kc"].copy(), h["vc"].copy()
            oatt.append_causal_kv(kc, vc, h["k"], h["v"], local, 0, s.cached, s.n_causal, 0, ps)
            assert np.array_equal(_f64(self.kc[h["pages"]]), kc), f"request {i}: appended K pages"
            assert np.array_equal(_f64(self.vc[h["pages"]]), vc), f"request {i}: appended V pages"
            K, Vv = oatt.gather_request_kv(kc, vc, h["k"], h["v"], local, 0, s.cached, s.n_causal, s.n_canvas, 0,
                                           ps)
            mask = oatt.visibility_mask(s.cached, s.n_causal, s.n_canvas)
            sel = np.arange(nr)
            rows = torch.as_tensor(int(self.lay.row0[i]) + sel, device="cuda")
            got = _f64(out[rows])
            for hq in range(self.Hq):
                ref = oatt.dense_mask_attention(h["q"][sel, hq], K[:, hq // G], Vv[:, hq // G], mask[sel],
                                                self.scale)
                err = float(np.abs(got[:, hq] - ref).max())
                worst = max(worst, err)
                assert err <= P.TOL_ATT_BF16, (i, hq, err)
        return worst


# ------------------------------------------------------------------ batched serving
def test_batched_attention_full_size():
    """32 requests, prefixes U{512..8192}, 256-row canvases; two requests in their commit pass
    (256 causal rows appended, no canvas rows); 16 query / 8 KV heads, head_dim 256."""
    torch = P.torch_mod()
    cfg = configs.BATCHED
    print("batched attention full size", flush=True)
    lay = synth.paged_layout(cfg["seed"], synth.batched_splits(cfg), cfg["page_size"], tag="batched.att")
    a = AttLaunch(lay, cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["seed"], "batched.att")
    longest = int(np.argmax([s.cached for s in lay.splits]))
    reqs = sorted({5, 21, 0, 13, 31, longest})   # the fp64 brute-force oracle takes ~30 s for the longest
    snap = a.snapshot(reqs)
    out = a.run()
    torch.cuda.synchronize()
    worst = a.check_all(out, reqs, snap)
    print(f"batched attention: max |delta| {worst:.3e} over every row of {len(reqs)} requests", flush=True)


def test_batched_sampler_accept_converged_full_size():
    """One global step of the batched workload: sampler over 32 x 256 rows of V = 262144 (the two
    requests in their commit pass inactive), then accept and converged on every canvas, with the
    staggered per-request steps of the workload."""
    import denoise_step_amd as dg
    torch = P.torch_mod()
    cfg = configs.BATCHED
    B, C, V = cfg["B"], cfg["C"], cfg["V"]
    print("batched sampler full size 8192 x 262144", flush=True)
    logits = synth.zipf_logits_torch(cfg["seed"], "batched.logits", B * C, V, "cuda")
    commit = (5, 21)
    active = np.array([0 if r in commit else 1 for r in range(B)], np.uint8)
    seeds = [(r << 32) | cfg["seed"] for r in range(B)]
    step_in_block = np.array([(2 * r) % cfg["max_steps"] for r in range(B)], np.int64)
    step_in_block[30] = cfg["max_steps"] - 1                 # this one reaches the cap now
    step_global = 2 * np.arange(B, dtype=np.int64) + 100
    out = dg.dg_denoise_sample(logits, V, C, P.dev(_i64(seeds)), P.dev(step_global.astype(np.int32)),
                               cfg["temperature"], active=P.dev(active))
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    rng = synth.rng_for(0, "batched.sampler.rows")
    rows = sorted(set(r * C + p for r in range(B) if active[r] for p in (0, 255)) |
                  set(r * C + int(p) for r in range(B) if active[r] for p in rng.choice(C, 6, replace=False)))
    host = _f64(logits[torch.as_tensor(rows, device="cuda")])
    ref = osamp.SampleOut(*(np.zeros(B * C) for _ in range(5)), argmax_gap=np.zeros(B * C),
                          key_gap=np.zeros(B * C))
    for i, r in enumerate(rows):
        req, pos = divmod(r, C)
        one = P.sampler_oracle_row(host[i], seeds[req], pos, int(step_global[req]))
        for f in ("entropy", "argmax", "sample", "row_max", "row_lnz", "argmax_gap", "key_gap"):
            getattr(ref, f)[r] = getattr(one, f)[0]
    P.check_sampler_rows({k: v[rows] for k, v in got.items()}, ref, rows)

    # accept: the GPU's own entropies and candidates, fed to both sides
    H = got["entropy"].reshape(B, C).copy()
    samp = got["sample"].reshape(B, C).copy()
    for r in commit:                                          # rows the sampler left unwritten
        H[r] = 0.0
        samp[r] = 0
    canvas0 = synth.rng_for(0, "batched.canvas").integers(0, V, (B, C)).astype(np.int32)
    canvas = P.dev(canvas0)
    acc = torch.zeros((B, C), dtype=torch.uint8, device="cuda")
    nacc = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    dg.dg_entropy_accept(P.dev(H), P.dev(samp), canvas, V, cfg["budget"], P.dev(_i64(seeds)),
                         P.dev(step_global.astype(np.int32)), active=P.dev(active), accept=acc, n_accept=nacc)
    aref = oacc.entropy_accept(H, samp, canvas0, cfg["budget"], seeds, step_global, V, active=active)
    gc, ga, gn = canvas.cpu().numpy(), acc.cpu().numpy(), nacc.cpu().numpy()
    for b in range(B):
        if not active[b]:
            assert np.array_equal(gc[b], canvas0[b]) and gn[b] == -1
            continue
        if aref.budget_gap[b] < P.BUDGET_TIE and gn[b] != aref.n_accept[b]:
            P.report_tie("budget")
            continue
        assert gn[b] == aref.n_accept[b] and np.array_equal(ga[b], aref.accept[b]), b
        assert np.array_equal(gc[b], aref.canvas[b]), b
    assert aref.n_accept[active == 1].max() > 0

    # converged: staggered states, the GPU's argmax and entropies
    am = got["argmax"].reshape(B, C).copy()
    prev = am.astype(np.int64).copy()
    prev[1::3, 7] += 1                                        # some canvases changed since the last step
    st = oconv.LoopState(canvas=gc.astype(np.int64), prev_argmax=prev, unchanged=np.arange(B, dtype=np.int64) % 4,
                         step_in_block=step_in_block.copy(), step_global=step_global.copy(),
                         sc_on=np.ones(B, np.uint8))
    i32 = lambda x: P.dev(np.asarray(x, np.int32))
    ds = dict(prev_argmax=i32(st.prev_argmax), unchanged=i32(st.unchanged), step_in_block=i32(st.step_in_block),
              step_global=i32(st.step_global), canvas=i32(st.canvas), sc_on=P.dev(st.sc_on),
              committed=torch.zeros(B, dtype=torch.uint8, device="cuda"),
              out_tokens=torch.zeros((B, C), dtype=torch.int32, device="cuda"),
              steps_used=torch.zeros(B, dtype=torch.int32, device="cuda"),
              num_sampled=torch.zeros(B, dtype=torch.int32, device="cuda"))
    cref = oconv.converged(am, H, st, cfg["k"], cfg["tau"], cfg["max_steps"], seeds, V, active=active)
    dg.dg_converged(P.dev(am.astype(np.int32)), P.dev(H), V, cfg["k"], cfg["tau"], cfg["max_steps"],
                    P.dev(_i64(seeds)), ds, active=P.dev(active))
    g2 = {k: v.cpu().numpy() for k, v in ds.items()}
    for b in range(B):
        if not active[b]:
            continue
        assert g2["committed"][b] == cref.committed[b], b
        assert g2["num_sampled"][b] == cref.num_sampled[b], b
        if cref.committed[b]:
            assert g2["steps_used"][b] == cref.steps_used[b], b
            assert np.array_equal(g2["out_tokens"][b], cref.out_tokens[b]), b
    for f in ("canvas", "prev_argmax", "unchanged", "step_in_block", "step_global", "sc_on"):
        assert np.array_equal(g2[f].astype(np.int64)[active == 1], getattr(st, f).astype(np.int64)[active == 1]), f
    assert cref.committed[30] == 1 and cref.committed.sum() >= 1


def test_batched_selfcond_full_size_two_rows_per_request():
    """P.E over 32 x 256 rows (the 8192-row launch: many M tiles, no split-K), MLP and embedding;
    self-conditioning on for some requests and off for others."""
    import denoise_step_amd as dg
    torch = P.torch_mod()
    cfg = configs.BATCHED
    B, C, V, d, hidden = cfg["B"], cfg["C"], cfg["V"], cfg["d"], cfg["hidden"]
    print("batched selfcond full size", flush=True)
    E = synth.normal_torch(0, "batched.E", (V, d), 1 / 8, torch.bfloat16, "cuda")
    wg = synth.normal_torch(0, "batched.wg", (d, hidden), 0.02, torch.bfloat16, "cuda")
    wu = synth.normal_torch(0, "batched.wu", (d, hidden), 0.02, torch.bfloat16, "cuda")
    wd = synth.normal_torch(0, "batched.wd", (hidden, d), 0.02, torch.bfloat16, "cuda")
    lt = synth.zipf_logits_torch(0, "batched.sc.logits", B * C, V, "cuda")
    st = dg.dg_denoise_sample(lt, V, C, P.dev(_i64([1] * B)), P.dev(np.zeros(B, np.int32)), 1.0)
    canvas = synth.rng_for(0, "batched.sc.canvas").integers(0, V, (B, C)).astype(np.int32)
    sc_on = (np.arange(B) % 3 != 0).astype(np.uint8)
    prepared = dg.dg_selfcond_prepare(E, wg, wu, wd)
    s_out = torch.empty((B * C, d), dtype=torch.float32, device="cuda")
    y_out = torch.empty((B * C, d), dtype=torch.float32, device="cuda")
    x = dg.dg_selfcond_embed(lt, V, st["row_max"], st["row_lnz"], P.dev(sc_on), P.dev(canvas), E, wg, wu, wd,
                             prepared, s_out=s_out, y_out=y_out)
    torch.cuda.synchronize()
    rng = synth.rng_for(0, "batched.sc.rows")
    rows = sorted(r * C + int(p) for r in range(B) for p in rng.choice(C, 2, replace=False))   # 2 per request
    idx = torch.as_tensor(rows, device="cuda")
    host_l = _f64(lt[idx])
    Pm = np.stack([osamp.probabilities(host_l[i], 1.0) for i in range(len(rows))])
    s_ref = P.oracle_pe_slabs(Pm, P.torch_table_rows(E), V)
    es = P.rel_norm_err(s_out[idx].cpu().numpy(), s_ref)
    assert es.max() <= P.TOL_NORM_REL, es
    y_ref = osc.gated_mlp(s_ref, _f64(wg), _f64(wu), _f64(wd))
    ey = P.rel_norm_err(y_out[idx].cpu().numpy(), y_ref)
    assert ey.max() <= P.TOL_NORM_REL, ey
    on = np.array([sc_on[r // C] for r in rows], np.float64)[:, None]
    x_ref = _f64(E[torch.as_tensor(canvas.reshape(-1)[rows].astype(np.int64), device="cuda")]) + on * y_ref
    P.check_bf16_output(_f64(x[idx]), x_ref)
    print(f"batched selfcond: P.E max normwise rel err {es.max():.2e}, MLP {ey.max():.2e}", flush=True)


# ------------------------------------------------------------------ structured read
def test_structured_read_attention_full_size():
    """64 requests, each a 2048-row causal prompt chunk (K/V appended, nothing cached before it)
    plus a 256-row canvas, 16 query / 8 KV heads, head_dim 256: causal tiles skip their fully
    masked key blocks; canvas rows see all 2304 keys."""
    torch = P.torch_mod()
    cfg = configs.STRUCTURED_READ
    print("structured-read attention full size", flush=True)
    lay = synth.paged_layout(cfg["seed"], synth.structured_read_splits(cfg), cfg["page_size"], tag="sread.att")
    a = AttLaunch(lay, cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["seed"], "sread.att")
    reqs = [0, 17, 63]                            # the fp64 brute-force oracle takes ~20 s per request
    snap = a.snapshot(reqs)
    out = a.run()
    torch.cuda.synchronize()
    worst = a.check_all(out, reqs, snap)
    print(f"structured-read attention: max |delta| {worst:.3e} over every row of {len(reqs)} requests", flush=True)


# ------------------------------------------------------------------ block draft
@pytest.mark.parametrize("layer", range(5))
def test_block_draft_attention_full_size(layer):
    """One of the five draft layers: 128 requests x 16 draft rows over injected context U{256..4096},
    32 query / 8 KV heads, head_dim 128 (each layer its own injected K/V)."""
    torch = P.torch_mod()
    cfg = configs.BLOCK_DRAFT
    print(f"block-draft attention layer {layer}", flush=True)
    tag = f"block_draft.att{layer}"
    lay = synth.paged_layout(cfg["seed"], synth.block_draft_splits(cfg), cfg["page_size"], tag=tag)
    a = AttLaunch(lay, cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["seed"], tag)
    out = a.run()
    torch.cuda.synchronize()
    worst = a.check_all(out, range(len(lay.splits)), {})   # no causal rows: pages unchanged by the launch
    print(f"block-draft layer {layer}: max |delta| {worst:.3e} over every row of all {len(lay.splits)} requests",
          flush=True)
