"""Pins for oracle.attention.

* the page's visibility examples (tests/golden/) fix the mask rule;
* an independent brute force: every key of every request laid out in one
  global list by inverting the page tables, visibility decided by a position
  predicate (same request and (canvas query or key position <= query
  position)), softmax written with -inf masking over the full score matrix;
* special cases with known outputs and invariances.
"""
import numpy as np
import pytest

import synth
from oracle import attention
from tests.golden.fixtures import read_blocks


def test_p0p1c0c1_fixture():
    blocks = read_blocks("visibility_p0p1c0c1.txt")
    _, rows = blocks[("mask", "p0p1c0c1")]
    assert attention.visibility_mask(0, 2, 2).astype(int).tolist() == rows


@pytest.mark.parametrize("fixture", ["visibility_three_requests.txt", "visibility_three_requests_window2.txt"])
def test_three_request_fixture_masks_and_tiles(fixture):
    blocks = read_blocks(fixture)
    for name in ("request0", "request1", "request2"):
        hdr, rows = blocks[("mask", name)]
        cached, nc, nv = (int(t) for t in hdr[0].split("=")[1].split(","))
        window = int(hdr[1].split("=")[1]) if len(hdr) > 1 else 0
        m = attention.visibility_mask(cached, nc, nv, window)
        assert m.astype(int).tolist() == rows
        if ("skipped_tiles", name) in blocks:
            _, tiles = blocks[("skipped_tiles", name)]
            tr, tc = -(-m.shape[0] // 2), -(-m.shape[1] // 2)
            skip = [[int(not m[2 * i:2 * i + 2, 2 * j:2 * j + 2].any()) for j in range(tc)] for i in range(tr)]
            assert skip == tiles


def _as_float(p, a):
    return synth.bf16_bits_to_f32(a).astype(np.float64) if p.dtype == "bf16" else a.astype(np.float64)


def brute_force(p, scale, window=0):
    """Global dense-mask attention over all requests (independent of the oracle's gather).

    With window W > 0 a key is visible only if its position is within W of the query's: at most W
    before it for a causal query, on either side for a canvas query."""
    q, k, v = _as_float(p, p.q), _as_float(p, p.k), _as_float(p, p.v)
    kc, vc = _as_float(p, p.k_cache), _as_float(p, p.v_cache)
    ps = p.page_size
    owner = {}                                    # physical page -> (request, logical page)
    for r, s in enumerate(p.splits):
        n = max(1, -(-(s.cached + s.n_causal) // ps))
        for lp in range(n):
            owner[int(p.page_table[p.page0[r] + lp])] = (r, lp)
    keys, vals, kreq, kpos, kcanvas = [], [], [], [], []
    for phys in range(kc.shape[0]):              # prefix keys straight from the physical pages
        if phys not in owner:
            continue
        r, lp = owner[phys]
        for slot in range(ps):
            pos = lp * ps + slot
            if pos < p.splits[r].cached:
                keys.append(kc[phys, :, slot]); vals.append(vc[phys, :, slot])
                kreq.append(r); kpos.append(pos); kcanvas.append(False)
    qreq, qpos, qcanvas = [], [], []
    for r, s in enumerate(p.splits):             # new rows: causal rows then canvas rows
        for j in range(s.n_causal + s.n_canvas):
            row = p.row0[r] + j
            is_canvas = j >= s.n_causal
            pos = s.cached + j
            keys.append(k[row]); vals.append(v[row]); kreq.append(r); kpos.append(pos); kcanvas.append(is_canvas)
            qreq.append(r); qpos.append(pos); qcanvas.append(is_canvas)
    K, Vv = np.stack(keys), np.stack(vals)        # [nk, Hkv, D]
    kreq, kpos = np.array(kreq), np.array(kpos)
    qreq, qpos, qcanvas = np.array(qreq), np.array(qpos), np.array(qcanvas)
    vis = (qreq[:, None] == kreq[None, :]) & (qcanvas[:, None] | (kpos[None, :] <= qpos[:, None]))
    if window > 0:
        dist = kpos[None, :] - qpos[:, None]
        vis &= (dist >= -window) & (qcanvas[:, None] | (dist <= 0)) & (dist <= window)
    group = p.Hq // p.Hkv
    out = np.zeros(q.shape)
    for h in range(p.Hq):
        sc = scale * q[:, h] @ K[:, h // group].T
        sc = np.where(vis, sc, -np.inf)
        w = np.exp(sc - sc.max(axis=1, keepdims=True))
        out[:, h] = (w / w.sum(axis=1, keepdims=True)) @ Vv[:, h // group]
    return out


def run_oracle(p, scale, window=0):
    f = lambda a: _as_float(p, a)
    splits = [(p.row0[i], s.cached, s.n_causal, s.n_canvas, p.page0[i], window) for i, s in enumerate(p.splits)]
    return attention.canvas_attention(f(p.q), f(p.k), f(p.v), f(p.k_cache), f(p.v_cache), p.page_table,
                                      splits, p.page_size, scale)


CASES = [
    ([(0, 6, 0), (6, 0, 4), (6, 4, 0)], 2, 1, 8),                 # the three-request batch
    ([(0, 2, 2)], 2, 2, 4),                                      # p0 p1 c0 c1
    ([(37, 0, 16), (5, 21, 3), (0, 17, 0), (64, 16, 0)], 4, 2, 16),
    ([(100, 0, 33)], 8, 2, 32),
]


@pytest.mark.parametrize("splits,Hq,Hkv,D", CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_oracle_matches_brute_force(splits, Hq, Hkv, D, dtype):
    p = synth.attention_problem(11, splits, Hq, Hkv, D, dtype=dtype)
    scale = 1.0 / np.sqrt(D)
    out, kc, _vc = run_oracle(p, scale)
    np.testing.assert_allclose(out, brute_force(p, scale), rtol=1e-12, atol=1e-12)
    # causal rows' K/V appended at cached + j, nothing else touched
    base = _as_float(p, p.k_cache)
    knew = _as_float(p, p.k)
    touched = np.zeros(base.shape[:1] + base.shape[2:3], bool)
    for r, s in enumerate(p.splits):
        for j in range(s.n_causal):
            pos = s.cached + j
            phys = p.page_table[p.page0[r] + pos // p.page_size]
            np.testing.assert_array_equal(kc[phys, :, pos % p.page_size], knew[p.row0[r] + j])
            touched[phys, pos % p.page_size] = True
    for phys in range(base.shape[0]):
        for slot in range(p.page_size):
            if not touched[phys, slot]:
                np.testing.assert_array_equal(kc[phys, :, slot], base[phys, :, slot])


def test_single_visible_key_returns_its_value():
    p = synth.attention_problem(3, [(0, 3, 0)], 2, 2, 8, dtype="f32")
    out, _, _ = run_oracle(p, 0.3)
    v = p.v.astype(np.float64)
    np.testing.assert_allclose(out[0], v[0], rtol=0, atol=1e-15)     # first causal row sees only itself


def test_equal_scores_average_visible_values():
    p = synth.attention_problem(4, [(5, 2, 3)], 2, 1, 8, dtype="f32")
    p.q[:] = 0.0                                                     # all scores equal
    out, kc, vc = run_oracle(p, 1.0)
    K, Vv = attention.gather_request_kv(kc, vc, p.k.astype(np.float64), p.v.astype(np.float64),
                                        p.page_table, 0, 5, 2, 3, 0, p.page_size)
    np.testing.assert_allclose(out[0, 0], Vv[:6, 0].mean(0), atol=1e-14)   # causal row 0 sees 5 + 1 keys
    np.testing.assert_allclose(out[4, 1], Vv[:, 0].mean(0), atol=1e-14)    # canvas row sees all 10


def test_canvas_row_permutation_and_prompt_isolation():
    p = synth.attention_problem(5, [(8, 4, 6)], 4, 2, 16, dtype="f32")
    out, _, _ = run_oracle(p, 0.25)
    perm = np.array([0, 1, 2, 3, 9, 7, 4, 8, 5, 6])
    p2 = synth.attention_problem(5, [(8, 4, 6)], 4, 2, 16, dtype="f32")
    p2.q, p2.k, p2.v = p.q[perm], p.k[perm], p.v[perm]
    out2, _, _ = run_oracle(p2, 0.25)
    np.testing.assert_allclose(out2, out[perm], atol=1e-13)
    p3 = synth.attention_problem(5, [(8, 4, 6)], 4, 2, 16, dtype="f32")
    p3.k[4:] = np.random.default_rng(0).normal(size=p3.k[4:].shape)   # change canvas K/V only
    p3.v[4:] = 7.0
    out3, _, _ = run_oracle(p3, 0.25)
    np.testing.assert_array_equal(out3[:4], out[:4])                 # prompt rows never see the canvas
    assert not np.allclose(out3[4:], out[4:])


def test_page_relabelling_invariance():
    p = synth.attention_problem(6, [(40, 3, 5), (17, 0, 2)], 4, 2, 8, dtype="f32")
    out, _, _ = run_oracle(p, 0.3)
    relabel = np.random.default_rng(1).permutation(p.k_cache.shape[0])
    p.k_cache = p.k_cache[np.argsort(relabel)]
    p.v_cache = p.v_cache[np.argsort(relabel)]
    p.page_table = relabel[p.page_table].astype(np.int32)
    out2, _, _ = run_oracle(p, 0.3)
    np.testing.assert_array_equal(out2, out)


@pytest.mark.parametrize("window", [1, 3, 17])
@pytest.mark.parametrize("splits,Hq,Hkv,D", CASES)
def test_oracle_window_matches_brute_force(splits, Hq, Hkv, D, window):
    p = synth.attention_problem(12, splits, Hq, Hkv, D, dtype="f32")
    scale = 1.0 / np.sqrt(D)
    out, _, _ = run_oracle(p, scale, window)
    np.testing.assert_allclose(out, brute_force(p, scale, window), rtol=1e-12, atol=1e-12)


def test_window_wider_than_request_is_full_attention():
    p = synth.attention_problem(13, [(9, 4, 5), (0, 3, 0)], 4, 2, 8, dtype="f32")
    full, _, _ = run_oracle(p, 0.4)
    wide, _, _ = run_oracle(p, 0.4, window=9 + 4 + 5)
    np.testing.assert_array_equal(wide, full)


def test_window_equal_scores_average_the_band():
    """q = 0 makes every visible score equal: each row returns the mean of its band's values."""
    p = synth.attention_problem(14, [(7, 2, 4)], 2, 1, 8, dtype="f32")
    p.q[:] = 0.0
    out, kc, vc = run_oracle(p, 1.0, window=2)
    _, Vv = attention.gather_request_kv(kc, vc, p.k.astype(np.float64), p.v.astype(np.float64),
                                        p.page_table, 0, 7, 2, 4, 0, p.page_size)
    np.testing.assert_allclose(out[0, 0], Vv[5:8, 0].mean(0), atol=1e-14)    # causal row at 7: keys 5..7
    np.testing.assert_allclose(out[1, 1], Vv[6:9, 0].mean(0), atol=1e-14)    # causal row at 8: keys 6..8
    np.testing.assert_allclose(out[2, 0], Vv[7:12, 0].mean(0), atol=1e-14)   # canvas row at 9: keys 7..11
    np.testing.assert_allclose(out[5, 0], Vv[10:13, 0].mean(0), atol=1e-14)  # canvas row at 12: keys 10..12


def test_window_left_edge_is_shared_by_both_row_kinds():
    """Only the right edge differs: a canvas row's band minus the keys after it is the causal band."""
    for cached, nc, nv, w in [(5, 3, 4, 2), (0, 6, 6, 1), (30, 0, 8, 5)]:
        m = attention.visibility_mask(cached, nc, nv, w)
        for j in range(nv):
            pos = cached + nc + j
            row = m[nc + j].copy()
            row[pos + 1:] = False
            ref = np.zeros_like(row)
            ref[max(0, pos - w):pos + 1] = True
            np.testing.assert_array_equal(row, ref)


@pytest.mark.parametrize("splits,Hq,Hkv,D", CASES)
def test_e4m3_cache_reduces_to_the_plain_oracle_on_representable_rows(splits, Hq, Hkv, D):
    """When every fresh K/V value is an exact E4M3 value times the scale, quantising on append is
    the identity, so the E4M3 oracle equals the plain oracle on the decoded cache, and the appended
    codes are the rows' own codes."""
    from oracle import fp8
    p = synth.attention_problem(15, splits, Hq, Hkv, D, dtype="f32")
    rng = np.random.default_rng(15)
    ks, vs = 2.0 ** -4, 2.0 ** -3
    kc8 = rng.integers(0, 0x7F, p.k_cache.shape).astype(np.uint8) | (rng.integers(0, 2, p.k_cache.shape) * 0x80).astype(np.uint8)
    vc8 = rng.integers(0, 0x7F, p.v_cache.shape).astype(np.uint8)
    k8 = rng.integers(0, 0x7F, p.k.shape).astype(np.uint8)
    v8 = rng.integers(0, 0x7F, p.v.shape).astype(np.uint8) | 0x80
    k, v = fp8.decode_table(k8, ks), fp8.decode_table(v8, vs)
    sp = [(p.row0[i], s.cached, s.n_causal, s.n_canvas, p.page0[i]) for i, s in enumerate(p.splits)]
    q = p.q.astype(np.float64)
    out8, kn, vn = attention.canvas_attention_e4m3(q, k, v, kc8, vc8, ks, vs, p.page_table, sp, p.page_size, 0.2)
    ref, rkc, rvc = attention.canvas_attention(q, k, v, fp8.decode_table(kc8, ks), fp8.decode_table(vc8, vs),
                                               p.page_table, sp, p.page_size, 0.2)
    np.testing.assert_allclose(out8, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(fp8.decode_table(kn, ks), rkc)
    np.testing.assert_array_equal(fp8.decode_table(vn, vs), rvc)


def test_e4m3_cache_keeps_the_launch_rows_unquantised():
    """A canvas row over an empty cache sees only this launch's rows, at input precision."""
    p = synth.attention_problem(16, [(0, 0, 5)], 2, 1, 8, dtype="f32")
    kc8 = np.zeros(p.k_cache.shape, np.uint8)
    out8, _, _ = attention.canvas_attention_e4m3(p.q, p.k, p.v, kc8, kc8, 0.5, 0.5, p.page_table,
                                                 [(0, 0, 0, 5, 0)], p.page_size, 0.3)
    ref, _, _ = attention.canvas_attention(p.q, p.k, p.v, p.k_cache, p.v_cache, p.page_table, [(0, 0, 0, 5, 0)],
                                           p.page_size, 0.3)
    np.testing.assert_allclose(out8, ref, rtol=1e-12, atol=1e-12)
