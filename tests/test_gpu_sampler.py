"""GPU parity of dg_denoise_sample against oracle.sampler (through the C ABI)."""
import numpy as np
import pytest

import synth
from oracle import sampler as osamp
from tests import parity as P

pytestmark = pytest.mark.gpu


def run_gpu(logits_t, V, rows_per_req, seeds, steps, T=1.0, argmax_only=False, active=None):
    import denoise_step_amd as dg
    torch = P.torch_mod()
    sd = P.dev(np.asarray(seeds, np.uint64).view(np.int64))
    st = P.dev(np.asarray(steps, np.int32))
    act = None if active is None else P.dev(np.asarray(active, np.uint8))
    out = dg.dg_denoise_sample(logits_t, V, rows_per_req, sd, st, T, active=act, argmax_only=argmax_only)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V,ld,T", [(4999, 5000, 1.0), (1024, 1024, 1.0), (20000, 20008, 0.7), (8, 8, 1.3),
                                    (1, 8, 1.0), (17, 24, 1.0), (16385, 16392, 1.0)])
def test_sampler_small(dtype, V, ld, T):
    print(f"sampler small dtype={dtype} V={V} ld={ld} T={T}", flush=True)
    rows, rpr = 24, 8
    base = synth.zipf_logits_f32(1, ("samp", V), rows, ld)
    base[:, V:] = 1e4                      # junk past V must never be read as a logit
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(base)
        t = P.dev_bf16(bits)
        host = synth.bf16_bits_to_f32(bits).astype(np.float64)[:, :V]
    else:
        t = P.dev(base)
        host = base.astype(np.float64)[:, :V]
    seeds = [(r << 32) | 5 for r in range(rows // rpr)]
    steps = [3, 0, 77]
    got = run_gpu(t, V, rpr, seeds, steps, T)
    ref = osamp.denoise_sample(host, T, seeds, steps, rpr)
    P.check_sampler_rows(got, ref, list(range(rows)))


def test_sampler_exact_ties_and_extremes():
    rows, V = 16, 3000
    rng = np.random.default_rng(5)
    base = rng.integers(-4, 4, (rows, V)).astype(np.float32)      # massive exact ties
    base[3] = 0.0                                                 # uniform row: H = ln V, argmax 0
    base[4] = -1e4
    base[4, 1234] = 3.0                                           # one-hot row: H = 0
    bits = synth.f32_to_bf16_bits(base)
    got = run_gpu(P.dev_bf16(bits), V, rows, [11], [4])
    ref = osamp.denoise_sample(synth.bf16_bits_to_f32(bits).astype(np.float64), 1.0, [11], [4], rows)
    P.check_sampler_rows(got, ref, list(range(rows)))
    assert got["argmax"][3] == 0 and abs(got["entropy"][3] - np.log(V)) < 1e-4
    assert got["argmax"][4] == 1234 and got["sample"][4] == 1234 and got["entropy"][4] < 1e-6


def test_sampler_most_rows():
    """The largest launch the row grid allows (65535 rows; the host rejects one more), short rows:
    every row's sampler outputs against the oracle."""
    import denoise_step_amd as dg
    rows, V, rpr = 65535, 24, 17
    print(f"sampler {rows} rows x {V}", flush=True)
    bits = synth.zipf_logits_bf16(3, "most_rows", rows, V + 8)[:, :V + 8]
    seeds = [(r << 32) | 9 for r in range(rows // rpr)]
    steps = [r % 11 for r in range(rows // rpr)]
    got = run_gpu(P.dev_bf16(bits), V, rpr, seeds, steps)
    ref = osamp.denoise_sample(synth.bf16_bits_to_f32(bits).astype(np.float64)[:, :V], 1.0, seeds, steps, rpr)
    P.check_sampler_rows(got, ref, list(range(rows)))
    with pytest.raises(dg.DGError):
        dg.dg_denoise_sample(P.dev_bf16(np.zeros((65536, 32), np.uint16)), 32, 16, P.dev(np.zeros(4096, np.int64)),
                             P.dev(np.zeros(4096, np.int32)))


def test_sampler_argmax_only_and_inactive():
    rows, rpr, V = 32, 8, 7000
    bits = synth.zipf_logits_bf16(2, "amax", rows, V)
    t = P.dev_bf16(bits)
    import denoise_step_amd as dg
    torch = P.torch_mod()
    keep = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    out = dict(argmax=keep)
    dg.dg_denoise_sample(t, V, rpr, None, None, 1.0, active=P.dev(np.array([1, 0, 1, 1], np.uint8)),
                         argmax_only=True, out=out)
    got = keep.cpu().numpy()
    ref = np.argmax(synth.bf16_bits_to_f32(bits), axis=1)
    assert np.array_equal(got[:8], ref[:8]) and np.array_equal(got[16:], ref[16:])
    assert np.all(got[8:16] == -7)                                # inactive request untouched


def test_sampler_single_canvas_full_size_all_rows():
    """256 x 262144 bf16 logits (one 256-token canvas), in the launch configuration the bench times:
    every row against the oracle."""
    V, C = 262144, 256
    print("sampler full size 256 x 262144", flush=True)
    bits = synth.zipf_logits_bf16(0, "single_canvas.logits", C, V)
    t = P.dev_bf16(bits)
    seeds, steps = [0], [17]
    got = run_gpu(t, V, C, seeds, steps)
    got2 = run_gpu(t, V, C, seeds, steps)
    for k in got:
        assert np.array_equal(got[k], got2[k]), f"{k} not bitwise deterministic"
    ref = osamp.denoise_sample(synth.bf16_bits_to_f32(bits).astype(np.float64), 1.0, seeds, steps, C)
    P.check_sampler_rows(got, ref, list(range(C)))
    # entropies spread over the recipe's range
    assert got["entropy"].min() < 1.0 and got["entropy"].max() > 9.0


def test_sampler_block_draft_argmax_full_size():
    """2048 rows x 151936 bf16 (128 requests x 16 draft positions), argmax only: every row."""
    torch = P.torch_mod()
    print("sampler argmax-only 2048 x 151936", flush=True)
    t = synth.zipf_logits_torch(0, "block_draft.logits", 2048, 151936, "cuda")
    import denoise_step_amd as dg
    out = dg.dg_denoise_sample(t, 151936, 16, None, None, 1.0, argmax_only=True)
    torch.cuda.synchronize()
    got = out["argmax"].cpu().numpy()
    # every row: numpy's argmax (first index of the maximum) of the same bf16 values, 256 rows at a time
    for r0 in range(0, 2048, 256):
        host = t[r0:r0 + 256].float().cpu().numpy().astype(np.float64)
        ref = np.argmax(host, axis=1)
        for i in np.nonzero(got[r0:r0 + 256] != ref)[0]:
            srt = np.sort(host[i])
            assert 0 < srt[-1] - srt[-2] < P.TIE_GAP, (r0 + i, got[r0 + i], int(ref[i]))
            P.report_tie("argmax_gap")
