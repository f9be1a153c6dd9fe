"""GPU parity of dg_canvas_attention against oracle.attention (through the C ABI)."""
import numpy as np
import pytest

import synth
from oracle import attention as oatt
from tests import parity as P

pytestmark = pytest.mark.gpu


def _f(p, a):
    return synth.bf16_bits_to_f32(a).astype(np.float64) if p.dtype == "bf16" else a.astype(np.float64)


def run_case(splits, Hq, Hkv, D, dtype, seed=0, check_cache=True, window=0, max_keys=None):
    import denoise_step_amd as dg
    torch = P.torch_mod()
    p = synth.attention_problem(seed, splits, Hq, Hkv, D, dtype=dtype)
    up = (lambda a: P.dev_bf16(a)) if dtype == "bf16" else (lambda a: P.dev(a))
    q, k, v, kc, vc = (up(a) for a in (p.q, p.k, p.v, p.k_cache, p.v_cache))
    sp = np.array([[p.row0[i], s.cached, s.n_causal, s.n_canvas, p.page0[i], window]
                   for i, s in enumerate(p.splits)], np.int32)
    max_rows = max(s.n_causal + s.n_canvas for s in p.splits)
    if max_keys is None:
        max_keys = max(s.cached + s.n_causal + s.n_canvas for s in p.splits)
    scale = 1.0 / np.sqrt(D)
    out = dg.dg_canvas_attention(q, k, v, kc, vc, P.dev(p.page_table), P.dev(sp), max_rows, max_keys, scale)
    torch.cuda.synchronize()
    ref, rkc, rvc = oatt.canvas_attention(_f(p, p.q), _f(p, p.k), _f(p, p.v), _f(p, p.k_cache), _f(p, p.v_cache),
                                          p.page_table, [tuple(r) for r in sp], p.page_size, scale)
    got = P.host_f64(out)
    tol = P.TOL_ATT_BF16 if dtype == "bf16" else P.TOL_ATT_F32
    err = np.abs(got - ref).max()
    assert err <= tol, f"max |delta| {err}"
    if check_cache:
        assert np.array_equal(P.host_f64(kc), rkc) and np.array_equal(P.host_f64(vc), rvc)
    return err


SMALL = [
    ([(0, 6, 0), (6, 0, 4), (6, 4, 0)], 2, 1, 32),                # the three-request batch
    ([(5, 0, 0), (0, 1, 0), (3, 0, 1), (20, 1, 1), (0, 0, 0)], 2, 2, 128),  # empty and one-row requests, G = 1
    ([(0, 2, 2)], 2, 2, 32),                                     # p0 p1 c0 c1
    ([(37, 0, 16), (5, 21, 3), (0, 17, 0), (64, 16, 0)], 4, 2, 64),
    ([(100, 0, 33)], 8, 2, 128),
    ([(300, 40, 70), (1, 0, 129)], 16, 8, 256),
    ([(0, 200, 56)], 32, 8, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_attention_small(case, dtype):
    splits, Hq, Hkv, D = SMALL[case]
    print(f"attention case={case} dtype={dtype}", flush=True)
    run_case(splits, Hq, Hkv, D, dtype, seed=case)


def test_attention_single_canvas_full_size():
    """One 256-row canvas over a 2048-token paged prefix, 16 query / 8 KV heads, head_dim 256, bf16."""
    print("attention full size single canvas", flush=True)
    run_case([(2048, 0, 256)], 16, 8, 256, "bf16", seed=7)


def test_attention_walk_with_empty_items():
    """More work items than the grid's 4096 workgroups, so workgroups walk several items: 48 requests
    of 1000 causal + 24 canvas rows, nothing cached, Hq = Hkv = 2, head_dim 128 -> 8 key splits per
    request and 6144 items, 2304 of them empty (early causal tiles see no key of the later splits).
    By the launch's item numbering, 1280 walks go from an item that prefetches its successor and 768
    from an empty item (which cannot), so both ways of starting an item run; every row against the
    oracle."""
    print("attention walk with empty items", flush=True)
    run_case([(0, 1000, 24)] * 48, 2, 2, 128, "bf16", seed=11)


def _many_requests(n):
    """n small mixed requests; every ninth one has a long cached prefix, so its keys are split."""
    return [((1500 + 37 * k) if k % 9 == 4 else (k * 13) % 70, k % 3, 1 + k % 5) for k in range(n)]


@pytest.mark.parametrize("n_req,Hq,Hkv,D", [
    (80, 4, 2, 256),    # beyond the 64 requests whose plans stay in registers at head size 256
    (100, 8, 2, 128),   # the second register group at head size 128
    (150, 8, 2, 128),   # beyond both groups: descriptors rescanned per item
])
def test_attention_many_requests(n_req, Hq, Hkv, D):
    """Launches of more requests than one wave's lanes: the kernel's item lookup from the two
    register groups and from the descriptors themselves; every row against the oracle."""
    print(f"attention many requests n_req={n_req} D={D}", flush=True)
    run_case(_many_requests(n_req), Hq, Hkv, D, "bf16", seed=n_req)


def test_attention_tiny_loop_shapes_f32():
    """The tiny loop's launches: 32-row causal prefill, 16-row canvas over 32, 16-row commit pass."""
    for sp in ([(0, 32, 0)], [(32, 0, 16)], [(32, 16, 0)]):
        run_case(sp, 2, 2, 32, "f32", seed=11)


@pytest.mark.parametrize("splits,Hq,Hkv,D", [
    ([(3000, 300, 50)], 16, 8, 256),          # causal rows appended while the keys are split (6 splits)
    ([(1500, 100, 20), (7, 9, 3)], 32, 8, 128),  # G = 4, 8 splits, a second short request
])
def test_attention_causal_rows_with_key_splits(splits, Hq, Hkv, D):
    print(f"attention causal + splits {splits} {Hq}/{Hkv}/{D}", flush=True)
    run_case(splits, Hq, Hkv, D, "bf16", seed=21)


@pytest.mark.parametrize("splits,Hq,Hkv,D", [
    ([(261120 - 12, 4, 8)], 2, 1, 128),          # the longest supported key span: 16 splits of 255 blocks
    ([(100000, 3, 5), (40, 2, 2)], 4, 2, 256),    # past one split's 1024 staged pages at head size 256
])
def test_attention_longest_prefix(splits, Hq, Hkv, D):
    """Prefixes so long that a request needs more key splits than its work-item target asks for (each
    split's page list staged in LDS holds 1024 pages): every row against the oracle, causal rows appended
    at the end of the long cache."""
    print(f"attention long prefix {splits[0][0]} keys D={D}", flush=True)
    run_case(splits, Hq, Hkv, D, "bf16", seed=31)


WINDOWED = [
    ([(0, 6, 0), (6, 0, 4), (6, 4, 0)], 2, 1, 32, 2, "f32"),      # the W = 2 three-request figure
    ([(0, 6, 0), (6, 0, 4), (6, 4, 0)], 2, 1, 128, 2, "bf16"),
    ([(37, 0, 16), (5, 21, 3), (0, 17, 0), (64, 16, 0)], 4, 2, 64, 5, "f32"),
    ([(300, 40, 70), (1, 0, 129)], 16, 8, 256, 33, "bf16"),      # band narrower than a key block
    ([(2048, 0, 256)], 16, 8, 256, 128, "bf16"),                # single canvas, W = 128
    ([(1000, 100, 200), (70, 0, 64)], 32, 8, 128, 300, "bf16"),  # G = 4, band wider than a tile's rows
    ([(100, 0, 33)], 8, 2, 128, 1000, "bf16"),                   # window wider than the request
]


@pytest.mark.parametrize("case", range(len(WINDOWED)))
def test_attention_sliding_window(case):
    splits, Hq, Hkv, D, W, dtype = WINDOWED[case]
    print(f"attention window case={case} W={W}", flush=True)
    run_case(splits, Hq, Hkv, D, dtype, seed=40 + case, window=W)


def test_attention_sliding_window_tight_key_bound():
    """max_keys_per_req given as the band span (rows + 2W), well under cached + rows: fewer, shorter
    key splits, and the last split takes the block its 64-alignment adds."""
    splits, W = [(5000, 0, 256), (3001, 64, 0)], 200
    span = max(s[1] + s[2] for s in splits) + 2 * W
    print(f"attention window tight bound span={span}", flush=True)
    run_case(splits, 16, 8, 256, "bf16", seed=51, window=W, max_keys=span)


K_SCALE, V_SCALE = 2.0 ** -4, 2.0 ** -3


def run_case_e4m3(splits, Hq, Hkv, D, seed=0, window=0):
    """dg_canvas_attention_e4m3 against oracle.attention.canvas_attention_e4m3: outputs within the bf16
    tolerance, the appended codes and every other cache byte identical."""
    import denoise_step_amd as dg
    torch = P.torch_mod()
    p = synth.attention_problem(seed, splits, Hq, Hkv, D, dtype="bf16")
    kc8 = synth.e4m3_table(seed, "att8.kc", p.k_cache.shape, 1.0, K_SCALE)
    vc8 = synth.e4m3_table(seed, "att8.vc", p.v_cache.shape, 1.0, V_SCALE)
    q, k, v = (P.dev_bf16(a) for a in (p.q, p.k, p.v))
    kcd, vcd = P.dev(kc8), P.dev(vc8)
    sp = np.array([[p.row0[i], s.cached, s.n_causal, s.n_canvas, p.page0[i], window]
                   for i, s in enumerate(p.splits)], np.int32)
    max_rows = max(s.n_causal + s.n_canvas for s in p.splits)
    max_keys = max(s.cached + s.n_causal + s.n_canvas for s in p.splits)
    scale = 1.0 / np.sqrt(D)
    out = dg.dg_canvas_attention_e4m3(q, k, v, kcd, vcd, K_SCALE, V_SCALE, P.dev(p.page_table), P.dev(sp), max_rows,
                                      max_keys, scale)
    torch.cuda.synchronize()
    f = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64)
    ref, rkc, rvc = oatt.canvas_attention_e4m3(f(p.q), f(p.k), f(p.v), kc8, vc8, K_SCALE, V_SCALE, p.page_table,
                                               [tuple(r) for r in sp], p.page_size, scale)
    err = np.abs(P.host_f64(out) - ref).max()
    assert err <= P.TOL_ATT_BF16, f"max |delta| {err}"
    assert np.array_equal(kcd.cpu().numpy(), rkc) and np.array_equal(vcd.cpu().numpy(), rvc)
    return err


E4M3_CASES = [
    ([(0, 6, 0), (6, 0, 4), (6, 4, 0)], 2, 1, 128, 0),            # the three-request batch
    ([(5, 0, 0), (0, 1, 0), (3, 0, 1), (20, 1, 1), (0, 0, 0)], 2, 2, 256, 1),  # empty / one-row requests, W = 1
    ([(37, 0, 16), (5, 21, 3), (0, 17, 0), (64, 16, 0)], 4, 2, 128, 0),
    ([(300, 40, 70), (1, 0, 129)], 16, 8, 256, 0),               # blocks straddling the cache end
    ([(100, 0, 33)], 8, 2, 128, 0),
    ([(0, 200, 56)], 32, 8, 128, 0),
    ([(1000, 100, 200), (70, 0, 64)], 32, 8, 128, 300),          # sliding window
    ([(3000, 300, 50)], 16, 8, 256, 0),                          # causal rows appended while keys are split
]


@pytest.mark.parametrize("case", range(len(E4M3_CASES)))
def test_attention_e4m3_cache(case):
    splits, Hq, Hkv, D, W = E4M3_CASES[case]
    print(f"attention e4m3 cache case={case}", flush=True)
    run_case_e4m3(splits, Hq, Hkv, D, seed=60 + case, window=W)


def test_attention_e4m3_cache_single_canvas_full_size():
    print("attention e4m3 cache full size single canvas", flush=True)
    run_case_e4m3([(2048, 0, 256)], 16, 8, 256, seed=67)
