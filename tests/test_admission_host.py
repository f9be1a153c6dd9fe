"""dg_deficit_admit (host code in libdg) against oracle.admission, iteration by iteration.

The admission decision is host logic with no GPU work, so it is checked here on the CPU: every
output (admitted count, deficit, tokens scheduled) must match the oracle exactly on the golden
trace and on seeded random traces, including decode work above the budget."""
import numpy as np
import pytest

from oracle import admission
from tests.test_oracle_admission import random_case, read_trace


def run_native(budget, decode, arrivals):
    import denoise_step_amd as dg
    tr = admission.Trace()
    queue, d = [], 0
    for t, dec in enumerate(decode):
        queue += [(pid, s) for pid, (ta, s) in enumerate(arrivals) if ta == t]
        n, d, tok = dg.dg_deficit_admit(budget, dec, [s for _, s in queue], d)
        tr.admitted.append([queue[i][0] for i in range(n)])
        queue = queue[n:]
        tr.tokens.append(tok)
        tr.deficit.append(d)
    return tr


def test_golden_trace_native():
    budget, arrivals, iters = read_trace()
    tr = run_native(budget, [it[0] for it in iters], arrivals)
    assert tr.tokens == [it[2] for it in iters] and tr.deficit == [it[3] for it in iters]


@pytest.mark.parametrize("seed", range(30))
def test_native_matches_oracle(seed):
    budget, decode, arrivals = random_case(np.random.default_rng(500 + seed), n_iter=200, n_pf=40)
    a = run_native(budget, decode, arrivals)
    b = admission.simulate(budget, decode, arrivals)
    assert (a.admitted, a.tokens, a.deficit) == (b.admitted, b.tokens, b.deficit)


def test_native_validation():
    import denoise_step_amd as dg
    for args in [(0, 0, [1], 0), (10, -1, [1], 0), (10, 0, [0], 0)]:
        with pytest.raises(dg.DGError):
            dg.dg_deficit_admit(*args)
    assert dg.dg_deficit_admit(10, 3, [], 5) == (0, 5, 3)     # nothing waits: deficit unchanged


def test_serving_loop_rejects_launch_beyond_its_row_pools():
    """The host check runs before any launch: a burst admitted at once under the admit-on-arrival
    policy needs more rows than pools sized for one prefill per iteration."""
    import torch

    import synth
    from denoise_step_amd.serving import ServingLoop
    from synth.configs import SERVING
    cfg = dict(SERVING, R=8, burst=8, P_min=4000, P_max=4000)
    sched = synth.serving_schedule_inputs(cfg)
    pools = {k: torch.zeros((sched["max_rows"], 1)) for k in ("q", "k", "v")}
    loop = ServingLoop(cfg, sched, pools, device="cpu", policy="arrival")
    with pytest.raises(ValueError, match="rows"):
        loop.step(0)
    assert 8 * 4000 > sched["max_rows"]

