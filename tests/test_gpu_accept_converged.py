"""dg_accept_converged (one launch) against dg_entropy_accept followed by dg_converged: every state
tensor, the canvas and the accept outputs bitwise equal after every step of a trajectory that
covers the prefill case, denoise steps, a convergence commit, a step-cap commit and an inactive
request."""
import numpy as np
import pytest

import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


def _state(torch, B, C):
    z = lambda shape, dt=torch.int32: torch.zeros(shape, dtype=dt, device="cuda")
    return dict(prev_argmax=z((B, C)), unchanged=z(B), step_in_block=torch.full((B,), -1, dtype=torch.int32,
                                                                             device="cuda"),
                step_global=z(B), canvas=z((B, C)), sc_on=z(B, torch.uint8), committed=z(B, torch.uint8),
                out_tokens=z((B, C)), steps_used=z(B), num_sampled=z(B))


@pytest.mark.parametrize("C", [16, 256, 300])
def test_accept_converged_matches_two_calls(C):
    import denoise_step_amd as dg
    torch = P.torch_mod()
    print(f"accept+converged C={C}", flush=True)
    B, V, k, tau, max_steps, budget = 4, 5000, 2, 0.5, 6, 3.0
    seed = P.dev(np.array([3, 5, 7, 11], np.int64))
    a, b = _state(torch, B, C), _state(torch, B, C)
    rng = synth.rng_for(0, "accept_converged", C)
    stable = rng.integers(0, V, (B, C)).astype(np.int32)
    for t in range(14):
        # request 0 keeps a stable argmax with low entropy (converges), request 1 changes every step
        # (step cap), request 2 is inactive on odd steps, request 3 is restarted to prefill at t = 5
        argmax = rng.integers(0, V, (B, C)).astype(np.int32)
        argmax[0] = stable[0]
        entropy = rng.random((B, C)).astype(np.float32) * np.array([0.1, 2.0, 1.0, 0.5], np.float32)[:, None]
        sample = rng.integers(0, V, (B, C)).astype(np.int32)
        active = np.array([1, 1, t % 2 == 0, 1], np.uint8)
        if t == 5:
            for st in (a, b):
                st["step_in_block"][3] = -1
        ent, smp, am, act = P.dev(entropy), P.dev(sample), P.dev(argmax), P.dev(active)
        acc_a = torch.zeros((B, C), dtype=torch.uint8, device="cuda")
        acc_b = torch.zeros((B, C), dtype=torch.uint8, device="cuda")
        na_a = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        na_b = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        # two calls: acceptance only for requests past their prefill case
        den = P.dev(((a["step_in_block"].cpu().numpy() >= 0) & (active == 1)).astype(np.uint8))
        step_now = a["step_global"].clone()
        dg.dg_entropy_accept(ent, smp, a["canvas"], V, budget, seed, step_now, active=den, accept=acc_a,
                             n_accept=na_a)
        dg.dg_converged(am, ent, V, k, tau, max_steps, seed, a, active=act)
        dg.dg_accept_converged(ent, smp, am, V, budget, k, tau, max_steps, seed, b, active=act, accept=acc_b,
                               n_accept=na_b)
        torch.cuda.synchronize()
        for key in a:
            assert torch.equal(a[key], b[key]), (t, key)
        assert torch.equal(acc_a, acc_b) and torch.equal(na_a, na_b), t
    steps_used = a["steps_used"].cpu().numpy()
    assert steps_used[0] > 0 and steps_used[1] == max_steps  # a convergence commit and a step-cap commit happened
