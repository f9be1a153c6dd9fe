"""The LM head fused with the sampler (dg_lmhead_denoise_sample) and P.E from its operand
(dg_selfcond_embed_lm) against the oracle's composition: backbone.lm_head (logits = scale h E^T in
fp64) -> sampler.denoise_sample -> selfcond.selfcond_embed.

Tolerances.  The fused path keeps the logits in fp32 (bf16 products accumulated by the MFMA over d
terms), so each logit carries an accumulation error of order sqrt(d / 16) 2^-24 |x|: about 2e-5 at
|x| = 25 for d = 4096, far below bf16's rounding of stored logits.  Outputs are checked as for the
sampler (entropy 1e-3, row_lnz 1e-4, s / y normwise 1e-3, x_next within a bf16 step) except that
row_max is compared at 1e-4 absolute, and an argmax or a sample that differs counts as a near-tie
(reported, not failed) only when the oracle's top-2 gap is below LM_TIE = 1e-3, fifty times the
accumulation error above.
"""
import numpy as np
import pytest

import synth
from oracle import backbone as obb
from oracle import sampler as osamp
from oracle import selfcond as osc
from synth import configs
from tests import parity as P

pytestmark = pytest.mark.gpu

LM_TIE = 1e-3


def check_lm_rows(got: dict, ref, rows):
    bad = []
    for i, r in enumerate(rows):
        if got["argmax"][i] != ref.argmax[r]:
            if ref.argmax_gap[r] < LM_TIE:
                P.report_tie("lmhead_argmax_gap")
            else:
                bad.append(("argmax", r, got["argmax"][i], ref.argmax[r], ref.argmax_gap[r]))
        if got["sample"][i] != ref.sample[r]:
            if ref.key_gap[r] < LM_TIE:
                P.report_tie("lmhead_key_gap")
            else:
                bad.append(("sample", r, got["sample"][i], ref.sample[r], ref.key_gap[r]))
        if abs(got["entropy"][i] - ref.entropy[r]) > P.TOL_ENTROPY:
            bad.append(("entropy", r, got["entropy"][i], ref.entropy[r]))
        if abs(got["row_max"][i] - ref.row_max[r]) > 1e-4:
            bad.append(("row_max", r, got["row_max"][i], ref.row_max[r]))
        if abs(got["row_lnz"][i] - ref.row_lnz[r]) > 1e-4:
            bad.append(("row_lnz", r, got["row_lnz"][i], ref.row_lnz[r]))
    assert not bad, bad[:10]


@pytest.mark.parametrize("B,C,V,d", [(2, 20, 16464, 256), (1, 300, 8192, 384), (3, 16, 40000, 128)])
def test_lmhead_small(B, C, V, d):
    """Ragged shapes: V = 16464 (two P.E runs, the second ragged; LM-head tiles with ids past V),
    300 rows (two row tiles, the second ragged), V = 40000 (three runs)."""
    import denoise_step_amd as dg
    torch = P.torch_mod()
    cfg = configs.LMHEAD_SMALL
    print(f"lmhead small B={B} C={C} V={V} d={d}", flush=True)
    rows, hidden = B * C, cfg["hidden"]
    tag = ("lmhead", B, C, V, d)
    E = synth.normal_bf16(cfg["seed"], tag + ("E",), (V, d), cfg["e_std"])
    h = synth.lmhead_hidden_bf16(cfg["seed"], tag, E, rows, cfg["a_max"] * 256 / d, cfg["b"])
    wg, wu = (synth.normal_bf16(cfg["seed"], tag + (t,), (d, hidden), cfg["w_std"]) for t in ("wg", "wu"))
    wd = synth.normal_bf16(cfg["seed"], tag + ("wd",), (hidden, d), cfg["w_std"])
    canvas = synth.rng_for(cfg["seed"], tag, "canvas").integers(0, V, (B, C)).astype(np.int32)
    sc_on = (np.arange(B) % 2 == 0).astype(np.uint8)
    seeds = np.arange(B, dtype=np.int64) * 977 + 3
    steps = np.arange(B, dtype=np.int32) + 4
    scale, T = cfg["scale"] * 256 / d, cfg["temperature"]
    Et, ht, wgt, wut, wdt = (P.dev_bf16(a) for a in (E, h, wg, wu, wd))
    st, op = dg.dg_lmhead_denoise_sample(ht, dg.dg_lmhead_prepare(Et), V, scale, C, P.dev(seeds), P.dev(steps), T)
    prepared = dg.dg_selfcond_prepare(Et, wgt, wut, wdt)
    s_out = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    y_out = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    x = dg.dg_selfcond_embed_lm(op, V, st["row_max"], st["row_lnz"], P.dev(sc_on), P.dev(canvas), Et, prepared,
                                hidden, s_out=s_out, y_out=y_out)
    torch.cuda.synchronize()

    f = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64)
    logits = obb.lm_head(f(h), f(E), scale)
    ref = osamp.denoise_sample(logits, T, seeds.astype(np.uint64), steps, C)
    check_lm_rows({k: v.cpu().numpy() for k, v in st.items()}, ref, list(range(rows)))
    H = ref.entropy
    print(f"entropy range {H.min():.3f} .. {H.max():.3f} nats")
    assert H.min() < 1.0 and H.max() > 5.0  # the recipe spans peaked and diffuse rows
    Pm = osc.probs_from_stats(logits, T, ref.row_max, ref.row_lnz)
    rx, rs, ry = osc.selfcond_embed(Pm, canvas, sc_on, f(E), f(wg), f(wu), f(wd), C, to_bf16=False)
    es = P.rel_norm_err(s_out.cpu().numpy(), rs)
    ey = P.rel_norm_err(y_out.cpu().numpy(), ry)
    print(f"lmhead operand: P.E max normwise rel err {es.max():.2e}, MLP {ey.max():.2e}")
    assert es.max() <= P.TOL_NORM_REL and ey.max() <= P.TOL_NORM_REL
    P.check_bf16_output(P.host_f64(x), rx)


def test_lmhead_inactive_rows_untouched():
    import denoise_step_amd as dg
    torch = P.torch_mod()
    print("lmhead inactive request", flush=True)
    B, C, V, d = 2, 16, 8192, 128
    E = synth.normal_bf16(5, "lmhead.inactive.E", (V, d), 1 / 8)
    h = synth.lmhead_hidden_bf16(5, "lmhead.inactive", E, B * C, 3.0, 0.125)
    out = dict(argmax=P.dev(np.full(B * C, -7, np.int32)), sample=P.dev(np.full(B * C, -7, np.int32)),
               entropy=P.dev(np.full(B * C, -7.0, np.float32)), row_max=P.dev(np.full(B * C, -7.0, np.float32)),
               row_lnz=P.dev(np.full(B * C, -7.0, np.float32)))
    seeds, steps = np.array([1, 2], np.int64), np.array([0, 0], np.int32)
    dg.dg_lmhead_denoise_sample(P.dev_bf16(h), dg.dg_lmhead_prepare(P.dev_bf16(E)), V, 8.0, C, P.dev(seeds),
                                P.dev(steps), 1.0, active=P.dev(np.array([0, 1], np.uint8)), out=out)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    for k, v in got.items():
        assert np.all(v[:C] == -7), k
    f = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64)
    ref = osamp.denoise_sample(obb.lm_head(f(h), f(E), 8.0), 1.0, seeds.astype(np.uint64), steps, C)
    check_lm_rows({k: v[C:] for k, v in got.items()}, ref, list(range(C, 2 * C)))


def test_lmhead_single_canvas_full_size_all_rows():
    """256 rows, V = 262144, d = 4096: every row's sampler outputs, s, y and x_next against the oracle
    composition (the fp64 logits and P.E computed over slabs of 16384 table rows)."""
    import denoise_step_amd as dg
    torch = P.torch_mod()
    cfg = configs.LMHEAD
    print("lmhead single canvas full size", flush=True)
    V, d, hidden, C = cfg["V"], cfg["d"], cfg["hidden"], cfg["C"]
    E = synth.normal_torch(0, "single_canvas.E", (V, d), cfg["e_std"], torch.bfloat16, "cuda")
    wg = synth.normal_torch(0, "single_canvas.wg", (d, hidden), cfg["w_std"], torch.bfloat16, "cuda")
    wu = synth.normal_torch(0, "single_canvas.wu", (d, hidden), cfg["w_std"], torch.bfloat16, "cuda")
    wd = synth.normal_torch(0, "single_canvas.wd", (hidden, d), cfg["w_std"], torch.bfloat16, "cuda")
    h = synth.lmhead_hidden_torch(0, "lmhead_single_canvas", E, C, cfg["a_max"], cfg["b"])
    canvas = P.dev(synth.rng_for(0, "single_canvas.canvas").integers(0, V, (1, C)).astype(np.int32))
    seeds, steps = np.array([11], np.int64), np.array([3], np.int32)
    on = P.dev(np.array([1], np.uint8))
    st, op = dg.dg_lmhead_denoise_sample(h, dg.dg_lmhead_prepare(E), V, cfg["scale"], C, P.dev(seeds), P.dev(steps),
                                         cfg["temperature"])
    prepared = dg.dg_selfcond_prepare(E, wg, wu, wd)
    s_out = torch.empty((C, d), dtype=torch.float32, device="cuda")
    y_out = torch.empty((C, d), dtype=torch.float32, device="cuda")
    x = dg.dg_selfcond_embed_lm(op, V, st["row_max"], st["row_lnz"], on, canvas, E, prepared, hidden, s_out=s_out,
                                y_out=y_out)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in st.items()}
    hh = h.float().cpu().numpy().astype(np.float64)
    slabs = [(v0, min(V, v0 + 16384)) for v0 in range(0, V, 16384)]
    logits = np.concatenate([obb.lm_head(hh, E[v0:v1].float().cpu().numpy().astype(np.float64), cfg["scale"])
                             for v0, v1 in slabs], axis=1)
    ref = osamp.denoise_sample(logits, cfg["temperature"], seeds.astype(np.uint64), steps, C)
    check_lm_rows(got, ref, list(range(C)))
    print(f"entropy range {ref.entropy.min():.3f} .. {ref.entropy.max():.3f} nats")
    Pm = osc.probs_from_stats(logits, cfg["temperature"], ref.row_max, ref.row_lnz)
    s_ref = P.oracle_pe_slabs(Pm, P.torch_table_rows(E), V)
    es = P.rel_norm_err(s_out.cpu().numpy(), s_ref)
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    y_ref = osc.gated_mlp(s_ref, f(wg), f(wu), f(wd))
    ey = P.rel_norm_err(y_out.cpu().numpy(), y_ref)
    print(f"lmhead full size, {C} rows against the oracle: s {es.max():.2e}, y {ey.max():.2e}")
    assert es.max() <= P.TOL_NORM_REL and ey.max() <= P.TOL_NORM_REL
    x_ref = f(E[canvas[0].long()]) + y_ref
    P.check_bf16_output(P.host_f64(x), x_ref)
