"""Batch invariance per request on the GPU: a request's outputs do not depend on the other
requests of a launch, on the launch's host bounds, or on which physical pages hold its cache.

Motivation: the single-pass-reads page (portfolio.ywsung.com), section on judging the saved launch
per request -- bf16 rounding that changes with the batch shape changes a request's answer.  The
library cuts a request's keys into attention splits, and a logit row into sampler chunks, from the
request's own shape only, so the comparisons here are bitwise.
"""
import numpy as np
import pytest

import synth
from synth import configs
from tests import parity as P

pytestmark = pytest.mark.gpu


def _layout():
    cfg = configs.BATCHED
    return cfg, synth.paged_layout(cfg["seed"], synth.batched_splits(cfg), cfg["page_size"], tag="inv.att")


def test_attention_alone_equals_in_batch_and_under_page_relabelling():
    """The 32-request batched launch (two requests in their commit pass) against single-request
    launches of five of its requests: bitwise equal outputs, also with looser host bounds and with
    the request's pages moved to other physical pages."""
    torch = P.torch_mod()
    import denoise_step_amd as dg
    cfg, lay = _layout()
    Hq, Hkv, D, ps = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["page_size"]
    print("attention batch invariance: 32-request batch", flush=True)
    bf = torch.bfloat16
    g = lambda name, shape: synth.normal_torch(7, ("inv", name), shape, 1.0, bf, "cuda")
    q, k, v = g("q", (lay.rows, Hq, D)), g("k", (lay.rows, Hkv, D)), g("v", (lay.rows, Hkv, D))
    kc0, vc0 = g("kc", (lay.n_pages, Hkv, ps, D)), g("vc", (lay.n_pages, Hkv, ps, D))
    scale = 1.0 / np.sqrt(D)
    max_rows = max(s.n_causal + s.n_canvas for s in lay.splits)
    max_keys = max(s.cached + s.n_causal + s.n_canvas for s in lay.splits)
    kc, vc = kc0.clone(), vc0.clone()
    out = dg.dg_canvas_attention(q, k, v, kc, vc, P.dev(lay.page_table), P.dev(lay.split_array()), max_rows,
                                 max_keys, scale)
    torch.cuda.synchronize()
    longest = int(np.argmax([s.cached for s in lay.splits]))
    for i in sorted({0, 5, 13, 21, longest}):
        s = lay.splits[i]
        r0, nr = int(lay.row0[i]), s.n_causal + s.n_canvas
        pages = lay.pages_of(i).astype(np.int64)
        nk = s.cached + nr
        sp = P.dev(np.array([[0, s.cached, s.n_causal, s.n_canvas, 0, 0]], np.int32))
        rows = slice(r0, r0 + nr)
        qi, ki, vi = q[rows].contiguous(), k[rows].contiguous(), v[rows].contiguous()
        for label, bounds, relabel in (("alone", (nr, nk), False), ("alone, loose bounds", (max_rows, max_keys), False),
                                       ("alone, pages relabelled", (nr, nk), True)):
            print(f"  request {i} ({s.cached} cached, {s.n_causal} causal, {s.n_canvas} canvas): {label}", flush=True)
            n_own = len(pages)
            if relabel:    # the request's pages at other physical slots of a larger cache, in reverse order
                perm = np.arange(n_own)[::-1] * 2 + 3
                kci = torch.zeros((2 * n_own + 4, Hkv, ps, D), dtype=bf, device="cuda")
                vci = torch.zeros_like(kci)
                kci[torch.as_tensor(perm, device="cuda")] = kc0[torch.as_tensor(pages, device="cuda")]
                vci[torch.as_tensor(perm, device="cuda")] = vc0[torch.as_tensor(pages, device="cuda")]
                table = perm.astype(np.int32)
            else:
                kci = kc0[torch.as_tensor(pages, device="cuda")].clone()
                vci = vc0[torch.as_tensor(pages, device="cuda")].clone()
                table = np.arange(n_own, dtype=np.int32)
            oi = dg.dg_canvas_attention(qi, ki, vi, kci, vci, P.dev(table), sp, bounds[0], bounds[1], scale)
            torch.cuda.synchronize()
            assert torch.equal(oi, out[rows]), (i, label)


def test_sampler_alone_equals_in_batch():
    """Eight 256-row canvases of V = 262144 logits (each request at its own step) against the same
    rows sampled one request at a time and in a batch of two: entropy, argmax, sample, row max and
    ln Z bitwise equal, for the plain and the fused-operand sampler."""
    torch = P.torch_mod()
    import denoise_step_amd as dg
    B, C, V = 8, 256, 262144
    print("sampler batch invariance: 8 x 256 rows of V = 262144", flush=True)
    logits = synth.zipf_logits_torch(3, "inv.logits", B * C, V, "cuda")
    seeds = torch.tensor([(5 << 20) + r for r in range(B)], dtype=torch.int64, device="cuda")
    steps = torch.tensor([3 * r + 1 for r in range(B)], dtype=torch.int32, device="cuda")
    names = ("entropy", "argmax", "sample", "row_max", "row_lnz")

    def run(rows, sd, st, sc):
        if sc:
            operand = torch.empty(dg.dg_selfcond_operand_bytes(rows.shape[0], V), dtype=torch.uint8, device="cuda")
            o, _ = dg.dg_denoise_sample_sc(rows, V, C, sd, st, 1.0, sc_operand=operand)
        else:
            o = dg.dg_denoise_sample(rows, V, C, sd, st, 1.0)
        torch.cuda.synchronize()
        return o

    for sc in (False, True):
        full = run(logits, seeds, steps, sc)
        for r in (0, 3, 7):
            alone = run(logits[r * C:(r + 1) * C], seeds[r:r + 1], steps[r:r + 1], sc)
            for n in names:
                assert torch.equal(alone[n], full[n][r * C:(r + 1) * C]), ("alone", sc, r, n)
        pair = run(logits[2 * C:4 * C], seeds[2:4], steps[2:4], sc)
        for n in names:
            assert torch.equal(pair[n], full[n][2 * C:4 * C]), ("pair", sc, n)
