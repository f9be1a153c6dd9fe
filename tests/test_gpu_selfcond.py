"""GPU parity of dg_selfcond_embed against oracle.selfcond (through the C ABI)."""
import numpy as np
import pytest

import synth
from oracle import sampler as osamp
from oracle import selfcond as osc
from tests import parity as P

pytestmark = pytest.mark.gpu


def _sampler_stats(logits_t, V, rows_per_req):
    import denoise_step_amd as dg
    n_req = logits_t.shape[0] // rows_per_req
    seeds = P.dev(np.arange(n_req, dtype=np.int64))
    steps = P.dev(np.zeros(n_req, np.int32))
    return dg.dg_denoise_sample(logits_t, V, rows_per_req, seeds, steps)


@pytest.mark.parametrize("V,d,hidden,w_std", [(1000, 128, 128, 0.02), (4096, 256, 384, 0.02), (2500, 128, 256, 0.5),
                                               (1000, 128, 128, 0.5)])
def test_selfcond_bf16_small(V, d, hidden, w_std):
    """w_std 0.5 makes the MLP output dominate x_out, so the normwise check exercises the MLP GEMMs."""
    import denoise_step_amd as dg
    torch = P.torch_mod()
    print(f"selfcond bf16 V={V} d={d} h={hidden}", flush=True)
    B, C = 3, 16
    rows = B * C
    ld = (V + 7) // 8 * 8
    L = synth.zipf_logits_f32(5, ("sc", V), rows, ld)
    bits = synth.f32_to_bf16_bits(L)
    E = synth.normal_bf16(5, ("sc.E", V), (V, d), 1 / 8)
    wg = synth.normal_bf16(5, ("sc.wg", V), (d, hidden), w_std)
    wu = synth.normal_bf16(5, ("sc.wu", V), (d, hidden), w_std)
    wd = synth.normal_bf16(5, ("sc.wd", V), (hidden, d), w_std)
    canvas = synth.rng_for(5, "sc.canvas").integers(0, V, (B, C)).astype(np.int32)
    sc_on = np.array([1, 0, 1], np.uint8)
    lt = P.dev_bf16(bits)
    Et, wgt, wut, wdt = (P.dev_bf16(a) for a in (E, wg, wu, wd))
    st = _sampler_stats(lt, V, C)
    prepared = dg.dg_selfcond_prepare(Et, wgt, wut, wdt)
    s_out = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    y_out = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    x = dg.dg_selfcond_embed(lt, V, st["row_max"], st["row_lnz"], P.dev(sc_on), P.dev(canvas), Et, wgt, wut, wdt,
                             prepared, s_out=s_out, y_out=y_out)
    torch.cuda.synchronize()
    host_l = synth.bf16_bits_to_f32(bits).astype(np.float64)[:, :V]
    ref = osamp.denoise_sample(host_l, 1.0, np.arange(B), np.zeros(B), C)
    Pm = osc.probs_from_stats(host_l, 1.0, ref.row_max, ref.row_lnz)
    f = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64)
    rx, rs, ry = osc.selfcond_embed(Pm, canvas, sc_on, f(E), f(wg), f(wu), f(wd), C, to_bf16=False)
    es = P.rel_norm_err(s_out.cpu().numpy(), rs)
    ey = P.rel_norm_err(y_out.cpu().numpy(), ry)
    print(f"P.E max normwise rel err {es.max():.2e}, MLP {ey.max():.2e}")
    assert es.max() <= P.TOL_NORM_REL, es.max()
    assert ey.max() <= P.TOL_NORM_REL, ey.max()
    gx = P.host_f64(x)
    P.check_bf16_output(gx, rx)
    on = np.repeat(sc_on.astype(bool), C)
    assert np.array_equal(gx[~on], f(E)[canvas.reshape(-1)][~on])       # self-conditioning off: plain lookup


@pytest.mark.parametrize("w_std", [0.02, 0.5])
def test_selfcond_f32_tiny_sizes(w_std):
    import denoise_step_amd as dg
    torch = P.torch_mod()
    B, C, V, d, hidden = 1, 16, 1024, 64, 128
    rows = B * C
    L = synth.zipf_logits_f32(6, "sc32", rows, V)
    E = synth.normal_f32(6, "sc32.E", (V, d), 1 / 8)
    w = [synth.normal_f32(6, t, sh, w_std) for t, sh in (("g", (d, hidden)), ("u", (d, hidden)), ("d", (hidden, d)))]
    canvas = synth.rng_for(6, "c").integers(0, V, (B, C)).astype(np.int32)
    lt = P.dev(L)
    st = _sampler_stats(lt, V, C)
    s_out = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    x = dg.dg_selfcond_embed(lt, V, st["row_max"], st["row_lnz"], P.dev(np.array([1], np.uint8)), P.dev(canvas),
                             P.dev(E), *(P.dev(a) for a in w), None, s_out=s_out)
    torch.cuda.synchronize()
    ref = osamp.denoise_sample(L.astype(np.float64), 1.0, [0], [0], C)
    Pm = osc.probs_from_stats(L.astype(np.float64), 1.0, ref.row_max, ref.row_lnz)
    rx, rs, ry = osc.selfcond_embed(Pm, canvas, np.array([1]), E, *w, C, to_bf16=False)
    assert P.rel_norm_err(s_out.cpu().numpy(), rs).max() <= 1e-5
    assert P.rel_norm_err(x.cpu().numpy(), rx).max() <= 1e-5


def test_selfcond_single_canvas_full_size_all_rows():
    """256 canvas rows, V = 262144, d = 4096, MLP 4096 -> 1024 -> 4096, in the bench's launch
    configuration: the sampler statistics, s = P.E, the MLP output y and x_next of every row
    against the oracle (fp64 P.E over slabs of the table)."""
    import denoise_step_amd as dg
    torch = P.torch_mod()
    print("selfcond full size, every row", flush=True)
    V, d, hidden, C = 262144, 4096, 1024, 256
    E = synth.normal_torch(0, "single_canvas.E", (V, d), 1 / 8, torch.bfloat16, "cuda")
    wg = synth.normal_torch(0, "single_canvas.wg", (d, hidden), 0.02, torch.bfloat16, "cuda")
    wu = synth.normal_torch(0, "single_canvas.wu", (d, hidden), 0.02, torch.bfloat16, "cuda")
    wd = synth.normal_torch(0, "single_canvas.wd", (hidden, d), 0.02, torch.bfloat16, "cuda")
    lt = synth.zipf_logits_torch(0, "single_canvas.logits_t", C, V, "cuda")
    canvas = synth.rng_for(0, "single_canvas.canvas").integers(0, V, (1, C)).astype(np.int32)
    st = _sampler_stats(lt, V, C)
    prepared = dg.dg_selfcond_prepare(E, wg, wu, wd)
    s_out = torch.empty((C, d), dtype=torch.float32, device="cuda")
    y_out = torch.empty((C, d), dtype=torch.float32, device="cuda")
    x = dg.dg_selfcond_embed(lt, V, st["row_max"], st["row_lnz"], P.dev(np.array([1], np.uint8)), P.dev(canvas), E,
                             wg, wu, wd, prepared, s_out=s_out, y_out=y_out)
    torch.cuda.synchronize()
    host_l = lt.float().cpu().numpy().astype(np.float64)
    ref = osamp.denoise_sample(host_l, 1.0, [0], [0], C)
    P.check_sampler_rows({k: v.cpu().numpy() for k, v in st.items()}, ref, list(range(C)))
    Pm = osc.probs_from_stats(host_l, 1.0, ref.row_max, ref.row_lnz)
    s_ref = P.oracle_pe_slabs(Pm, P.torch_table_rows(E), V)
    es = P.rel_norm_err(s_out.cpu().numpy(), s_ref)
    assert es.max() <= P.TOL_NORM_REL, es.max()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    y_ref = osc.gated_mlp(s_ref, f(wg), f(wu), f(wd))
    ey = P.rel_norm_err(y_out.cpu().numpy(), y_ref)
    print(f"full size, {C} rows: P.E max normwise rel err {es.max():.2e}, MLP {ey.max():.2e}")
    assert ey.max() <= P.TOL_NORM_REL, ey.max()
    x_ref = f(E[torch.as_tensor(canvas[0].astype(np.int64), device="cuda")]) + y_ref
    P.check_bf16_output(P.host_f64(x), x_ref)


@pytest.mark.parametrize("V,d,hidden,rows_per_req", [(1000, 128, 128, 16), (40000, 256, 256, 16),
                                                      (70000, 128, 384, 48)])
def test_selfcond_operand_from_sampler(V, d, hidden, rows_per_req):
    """dg_denoise_sample_sc writes the probability operand in 16384-id runs (the last one ragged);
    dg_selfcond_embed_sc must give the oracle's s, y and x_next, and the sampler outputs the oracle's."""
    import denoise_step_amd as dg
    torch = P.torch_mod()
    print(f"selfcond operand path V={V} d={d} h={hidden}", flush=True)
    B = 3
    C = rows_per_req
    rows = B * C
    ld = (V + 7) // 8 * 8
    L = synth.zipf_logits_f32(7, ("scop", V), rows, ld)
    bits = synth.f32_to_bf16_bits(L)
    E = synth.normal_bf16(7, ("scop.E", V), (V, d), 1 / 8)
    wg, wu = (synth.normal_bf16(7, (t, V), (d, hidden), 0.5) for t in ("scop.wg", "scop.wu"))
    wd = synth.normal_bf16(7, ("scop.wd", V), (hidden, d), 0.5)
    canvas = synth.rng_for(7, "scop.canvas").integers(0, V, (B, C)).astype(np.int32)
    sc_on = np.array([1, 0, 1], np.uint8)
    lt = P.dev_bf16(bits)
    Et, wgt, wut, wdt = (P.dev_bf16(a) for a in (E, wg, wu, wd))
    seeds = P.dev(np.arange(B, dtype=np.int64))
    steps = P.dev(np.full(B, 5, np.int32))
    st, op = dg.dg_denoise_sample_sc(lt, V, C, seeds, steps)
    prepared = dg.dg_selfcond_prepare(Et, wgt, wut, wdt)
    s_out = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    y_out = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    x = dg.dg_selfcond_embed_sc(op, V, st["row_max"], st["row_lnz"], P.dev(sc_on), P.dev(canvas), Et, prepared,
                                hidden, s_out=s_out, y_out=y_out)
    torch.cuda.synchronize()
    host_l = synth.bf16_bits_to_f32(bits).astype(np.float64)[:, :V]
    ref = osamp.denoise_sample(host_l, 1.0, np.arange(B), np.full(B, 5), C)
    got = {k: v.cpu().numpy() for k, v in st.items()}
    P.check_sampler_rows(got, ref, list(range(rows)))
    Pm = osc.probs_from_stats(host_l, 1.0, ref.row_max, ref.row_lnz)
    f = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64)
    rx, rs, ry = osc.selfcond_embed(Pm, canvas, sc_on, f(E), f(wg), f(wu), f(wd), C, to_bf16=False)
    es = P.rel_norm_err(s_out.cpu().numpy(), rs)
    ey = P.rel_norm_err(y_out.cpu().numpy(), ry)
    print(f"operand path: P.E max normwise rel err {es.max():.2e}, MLP {ey.max():.2e}")
    assert es.max() <= P.TOL_NORM_REL, es.max()
    assert ey.max() <= P.TOL_NORM_REL, ey.max()
    P.check_bf16_output(P.host_f64(x), rx)


def test_selfcond_operand_path_single_canvas_full_size():
    """The bench's fused pair at full size against the path that reads the logits again."""
    import denoise_step_amd as dg
    torch = P.torch_mod()
    print("selfcond operand path full size", flush=True)
    V, d, hidden, C = 262144, 4096, 1024, 256
    E = synth.normal_torch(0, "single_canvas.E", (V, d), 1 / 8, torch.bfloat16, "cuda")
    wg = synth.normal_torch(0, "single_canvas.wg", (d, hidden), 0.02, torch.bfloat16, "cuda")
    wu = synth.normal_torch(0, "single_canvas.wu", (d, hidden), 0.02, torch.bfloat16, "cuda")
    wd = synth.normal_torch(0, "single_canvas.wd", (hidden, d), 0.02, torch.bfloat16, "cuda")
    lt = synth.zipf_logits_torch(0, "single_canvas.logits_t", C, V, "cuda")
    canvas = P.dev(synth.rng_for(0, "single_canvas.canvas").integers(0, V, (1, C)).astype(np.int32))
    seeds, steps = P.dev(np.zeros(1, np.int64)), P.dev(np.zeros(1, np.int32))
    on = P.dev(np.array([1], np.uint8))
    st_a = dg.dg_denoise_sample(lt, V, C, seeds, steps)
    st_b, op = dg.dg_denoise_sample_sc(lt, V, C, seeds, steps)
    prepared = dg.dg_selfcond_prepare(E, wg, wu, wd)
    outs = []
    for path in ("logits", "operand"):
        s_out = torch.empty((C, d), dtype=torch.float32, device="cuda")
        y_out = torch.empty((C, d), dtype=torch.float32, device="cuda")
        if path == "logits":
            x = dg.dg_selfcond_embed(lt, V, st_a["row_max"], st_a["row_lnz"], on, canvas, E, wg, wu, wd, prepared,
                                     s_out=s_out, y_out=y_out)
        else:
            x = dg.dg_selfcond_embed_sc(op, V, st_b["row_max"], st_b["row_lnz"], on, canvas, E, prepared, hidden,
                                        s_out=s_out, y_out=y_out)
        outs.append((s_out, y_out, x))
    torch.cuda.synchronize()
    for k in ("argmax", "sample"):
        assert torch.equal(st_a[k], st_b[k]), k
    assert (st_a["entropy"] - st_b["entropy"]).abs().max().item() <= P.TOL_ENTROPY
    es = P.rel_norm_err(outs[1][0].cpu().numpy(), outs[0][0].cpu().numpy().astype(np.float64))
    ey = P.rel_norm_err(outs[1][1].cpu().numpy(), outs[0][1].cpu().numpy().astype(np.float64))
    print(f"operand vs logits path: s {es.max():.2e}, y {ey.max():.2e}")
    assert es.max() <= P.TOL_NORM_REL and ey.max() <= P.TOL_NORM_REL
    # every row against the oracle: the sampler outputs, s, y and x_next
    host_l = lt.float().cpu().numpy().astype(np.float64)
    ref = osamp.denoise_sample(host_l, 1.0, [0], [0], C)
    P.check_sampler_rows({k: v.cpu().numpy() for k, v in st_b.items()}, ref, list(range(C)))
    Pm = osc.probs_from_stats(host_l, 1.0, ref.row_max, ref.row_lnz)
    s_ref = P.oracle_pe_slabs(Pm, P.torch_table_rows(E), V)
    es = P.rel_norm_err(outs[1][0].cpu().numpy(), s_ref)
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    y_ref = osc.gated_mlp(s_ref, f(wg), f(wu), f(wd))
    ey = P.rel_norm_err(outs[1][1].cpu().numpy(), y_ref)
    print(f"operand path, {C} rows against the oracle: s {es.max():.2e}, y {ey.max():.2e}")
    assert es.max() <= P.TOL_NORM_REL and ey.max() <= P.TOL_NORM_REL
    x_ref = f(E[canvas[0].long()]) + y_ref
    P.check_bf16_output(P.host_f64(outs[1][2]), x_ref)
