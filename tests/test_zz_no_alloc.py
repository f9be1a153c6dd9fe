"""The allocation-free sampler entry point against the workspace one, through the C ABI.

dg_denoise_sample_noalloc keeps its chunk partials in the library's fixed per-device scratch
array; it must give exactly dg_denoise_sample's outputs.  Two calls in a row share the array, the
second with a smaller input (fewer rows, a shorter vocabulary, an argmax-only pass), so stale
partials of the first call must not leak into the second.
"""
import pytest

import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


def test_noalloc_sampler_matches_workspace_entry_point():
    torch = P.torch_mod()
    import denoise_step_amd as dg
    names = ("entropy", "argmax", "sample", "row_max", "row_lnz")
    for rows, V, rpr, amax_only in ((512, 262144, 256, False), (96, 50000, 32, False), (40, 20000, 8, True)):
        print(f"noalloc sampler: {rows} rows, V={V}, argmax_only={amax_only}", flush=True)
        logits = synth.zipf_logits_torch(11, ("noalloc", rows, V), rows, V, "cuda")
        n_req = rows // rpr
        seeds = torch.tensor([(9 << 24) + r for r in range(n_req)], dtype=torch.int64, device="cuda")
        steps = torch.tensor([7 * r for r in range(n_req)], dtype=torch.int32, device="cuda")
        ref = dg.dg_denoise_sample(logits, V, rpr, seeds, steps, 1.0, argmax_only=amax_only)
        out = {n: torch.full_like(ref[n], -7) for n in ref}
        torch.cuda.synchronize()
        dg.dg_denoise_sample_noalloc(logits, V, rpr, seeds, steps, out, 1.0, argmax_only=amax_only)
        torch.cuda.synchronize()
        for n in (("argmax",) if amax_only else names):
            assert torch.equal(out[n], ref[n]), (rows, V, n)
