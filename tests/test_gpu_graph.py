"""The bf16 denoise step (attention -> fused sampler -> acceptance + convergence -> self-conditioning)
captured into HIP graphs through torch's stream capture and replayed: every replay must reproduce,
bitwise, the state and outputs of the same step run eagerly from the same starting state.  The step
records no memset or copy nodes (every buffer is written by kernels), and the replays run with eager
work and synchronisations between them."""
import sys
import os

import pytest

from tests import parity as P

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _snapshot(w):
    keep = dict(w.state)
    keep.update(x=w.x, att=w.att_out, accept=w.accept, n_accept=w.n_accept, **{f"so_{k}": v for k, v in w.so.items()})
    return {k: v.clone() for k, v in keep.items()}


def _restore(w, snap):
    for k, v in w.state.items():
        v.copy_(snap[k])


def test_step_graph_replays_match_eager():
    torch = P.torch_mod()
    sys.path.insert(0, ROOT)
    import bench
    print("graph capture of the step (small shapes)", flush=True)
    cfg = dict(bench.CFG, C=64, L=256, V=16384, d=512, hidden=256, pool=3)
    w = bench.Workload(cfg)
    start = _snapshot(w)
    steps = 5
    eager = []
    for t in range(steps):
        w.step(t)
        torch.cuda.synchronize()
        eager.append(_snapshot(w))
    _restore(w, start)
    torch.cuda.synchronize()
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(cfg["pool"]):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                w.step(i)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    _restore(w, start)   # capture does not run the kernels, but leave no doubt about the starting state
    torch.cuda.synchronize()
    for t in range(steps):
        graphs[t % cfg["pool"]].replay()
        torch.cuda.synchronize()
        got = _snapshot(w)
        for k, ref in eager[t].items():
            assert torch.equal(got[k], ref), (t, k)
        torch.zeros(1 << 20, device="cuda").sum().item()   # eager work between replays
