"""GPU parity of the per-canvas state steps (Philox, accept, converged) and the small readouts."""
import numpy as np
import pytest

import synth
from oracle import accept as oacc
from oracle import converged as oconv
from oracle import philox, readout, verify
from tests import parity as P

pytestmark = pytest.mark.gpu


def i64(a):
    return np.asarray(a, np.uint64).view(np.int64)


def test_philox_device_matches_oracle():
    import denoise_step_amd as dg
    rng = synth.rng_for(0, "philox-kat")
    n = 20000
    ctr = rng.integers(0, 2 ** 32, (n, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2 ** 32, (n, 2), dtype=np.uint64).astype(np.uint32)
    ctr[:4] = 0
    key[:2] = 0
    ctr[4:8] = 0xFFFFFFFF
    out = dg.dg_philox4x32_10(P.dev(ctr.view(np.int32)), P.dev(key.view(np.int32)))
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, philox.philox4x32_10(ctr, key))


@pytest.mark.parametrize("C", [1, 16, 64, 65, 100, 256, 300, 512, 1000, 1024])  # every workgroup size, both sides of its edges
def test_entropy_accept_matches_oracle(C):
    import denoise_step_amd as dg
    torch = P.torch_mod()
    print(f"accept C={C}", flush=True)
    B, V = 6, 262144
    rng = synth.rng_for(1, "accept", C)
    H = rng.gamma(1.0, 2.0, (B, C)).astype(np.float32)
    H[1] = np.round(H[1] * 4) / 4                       # exact ties in entropy
    H[2, : C // 2] = 0.0
    H[3] = rng.uniform(0, 0.05, C).astype(np.float32)   # nearly all accepted
    sample = rng.integers(0, V, (B, C)).astype(np.int32)
    canvas0 = rng.integers(0, V, (B, C)).astype(np.int32)
    seeds = [(b << 32) | 9 for b in range(B)]
    steps = rng.integers(0, 1000, B).astype(np.int32)
    active = np.array([1, 1, 1, 1, 0, 1], np.uint8)
    for budget in (8.0, 2.0, 0.0, 1e9):
        canvas = P.dev(canvas0)
        acc = torch.zeros((B, C), dtype=torch.uint8, device="cuda")
        nacc = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        dg.dg_entropy_accept(P.dev(H), P.dev(sample), canvas, V, budget, P.dev(i64(seeds)), P.dev(steps),
                             active=P.dev(active), accept=acc, n_accept=nacc)
        ref = oacc.entropy_accept(H, sample, canvas0, budget, seeds, steps, V, active=active)
        gc, ga, gn = canvas.cpu().numpy(), acc.cpu().numpy(), nacc.cpu().numpy()
        for b in range(B):
            if not active[b]:
                assert np.array_equal(gc[b], canvas0[b]) and gn[b] == -1
                continue
            if ref.budget_gap[b] < P.BUDGET_TIE and gn[b] != ref.n_accept[b]:
                P.report_tie("budget")
                continue
            assert gn[b] == ref.n_accept[b], (budget, b)
            assert np.array_equal(ga[b], ref.accept[b]), (budget, b)
            assert np.array_equal(gc[b], ref.canvas[b]), (budget, b)


def _state_dev(st: oconv.LoopState, B, C):
    torch = P.torch_mod()
    i32 = lambda a: P.dev(np.asarray(a, np.int32))
    return dict(prev_argmax=i32(st.prev_argmax), unchanged=i32(st.unchanged), step_in_block=i32(st.step_in_block),
                step_global=i32(st.step_global), canvas=i32(st.canvas), sc_on=P.dev(np.asarray(st.sc_on, np.uint8)),
                committed=torch.zeros(B, dtype=torch.uint8, device="cuda"),
                out_tokens=torch.zeros((B, C), dtype=torch.int32, device="cuda"),
                steps_used=torch.zeros(B, dtype=torch.int32, device="cuda"),
                num_sampled=torch.zeros(B, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("C", [16, 256, 1000])
def test_converged_lockstep_histories(C):
    """Same generated argmax/entropy histories fed to both sides for 90 steps; state compared every step."""
    import denoise_step_amd as dg
    print(f"converged C={C}", flush=True)
    B, V, k, tau, max_steps = 5, 1000, 3, 0.3, 20
    rng = synth.rng_for(2, "conv", C)
    st = oconv.LoopState(canvas=np.zeros((B, C), np.int64), prev_argmax=np.zeros((B, C), np.int64),
                         unchanged=np.zeros(B, np.int64), step_in_block=np.array([-1, -1, 0, 5, -1]),
                         step_global=np.array([0, 7, 3, 100, 0]), sc_on=np.zeros(B, np.uint8))
    seeds = [(b << 32) | 4 for b in range(B)]
    ds = _state_dev(st, B, C)
    base = rng.integers(0, V, (B, C))
    for t in range(90):
        am = base.copy()
        am[1] = rng.integers(0, V, C)                   # always changing -> cap
        if t % 11 == 0:
            am[2, 0] += 1                               # occasional change
        H = np.where(np.arange(B)[:, None] == 3, 0.05, 0.1).astype(np.float32) * np.ones((B, C), np.float32)
        H[4] = rng.uniform(0, 0.6, C).astype(np.float32)
        active = np.array([1, 1, 1, 1, t % 3 != 0], np.uint8)
        ref = oconv.converged(am, H, st, k, tau, max_steps, seeds, V, active=active)
        dg.dg_converged(P.dev(am.astype(np.int32)), P.dev(H), V, k, tau, max_steps, P.dev(i64(seeds)), ds,
                        active=P.dev(active))
        got = {kk: v.cpu().numpy() for kk, v in ds.items()}
        for b in range(B):
            if not active[b]:
                continue
            if ref.mean_gap[b] < P.MEAN_TIE and got["committed"][b] != ref.committed[b]:
                # a mean entropy within 1e-3 of tau: counted; the oracle continues from the GPU's state
                P.report_tie("mean_entropy")
                for f in ("canvas", "prev_argmax", "unchanged", "step_in_block", "step_global", "sc_on"):
                    getattr(st, f)[b] = got[f][b]
                continue
            assert got["committed"][b] == ref.committed[b], (t, b)
            assert got["num_sampled"][b] == ref.num_sampled[b], (t, b)
            if ref.committed[b]:
                assert got["steps_used"][b] == ref.steps_used[b], (t, b)
                assert np.array_equal(got["out_tokens"][b], ref.out_tokens[b]), (t, b)
        for f in ("canvas", "prev_argmax", "unchanged", "step_in_block", "step_global", "sc_on"):
            assert np.array_equal(got[f].astype(np.int64), getattr(st, f).astype(np.int64)), (t, f)


def test_verify_prefix_block_draft_shape():
    import denoise_step_amd as dg
    B, L, V = 128, 16, 151936
    rng = synth.rng_for(3, "verify")
    draft = rng.integers(0, V, (B, L)).astype(np.int32)
    g = rng.geometric(0.2, B) - 1
    target = draft.copy()
    for b in range(B):
        if g[b] < L:
            target[b, g[b]] = (draft[b, g[b]] + 1 + rng.integers(0, V - 1)) % V
            target[b, g[b] + 1:] = rng.integers(0, V, L - 1 - g[b])
    got = dg.dg_verify_prefix(P.dev(draft), P.dev(target)).cpu().numpy()
    assert np.array_equal(got, verify.verify_prefix(draft, target))
    assert np.array_equal(got, np.minimum(g, L))


@pytest.mark.parametrize("V,full", [(5000, False), (262144, True)])
def test_allowed_probs_structured_read(V, full):
    """64 requests x 8 slots, 2-5 allowed ids each; slot rows are Philox-chosen canvas rows."""
    import denoise_step_amd as dg
    torch = P.torch_mod()
    print(f"allowed_probs V={V}", flush=True)
    B, C, slots = 64, 256, 8
    rng = synth.rng_for(4, "slots", V)
    counts = rng.integers(2, 6, B * slots)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ids = np.concatenate([rng.choice(V, c, replace=False) for c in counts]).astype(np.int32)
    n_rows = B * slots if full else 64
    slot_row = (np.arange(B * slots) % n_rows).astype(np.int32)
    if full:
        t = synth.zipf_logits_torch(4, "slots.logits", n_rows, V, "cuda")
    else:
        t = P.dev_bf16(synth.zipf_logits_bf16(4, "slots.logits", n_rows, V))
    ids[:2] = ids[2]                                    # duplicated id: equal logits -> first listed wins
    q, ans = dg.dg_allowed_probs(t, V, P.dev(slot_row), P.dev(offsets), P.dev(ids))
    host = t.float().cpu().numpy().astype(np.float64)[slot_row]
    rq, rans, gap = readout.allowed_probs(host, offsets, ids)
    gq = q.cpu().numpy()
    np.testing.assert_allclose(gq, rq, rtol=P.TOL_PROB_REL, atol=1e-7)
    ga = ans.cpu().numpy()
    for s in range(B * slots):
        if ga[s] != rans[s]:
            assert 0 < gap[s] < P.TIE_GAP
            P.report_tie("allowed_argmax")
