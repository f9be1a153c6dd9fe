"""Pins for oracle.sampler: entropy closed forms, softmax/argmax identities, Gumbel-max law."""
import math

import numpy as np
import pytest
from scipy import stats

import synth
from oracle import sampler

NEG = -1.0e4  # exp(NEG - max) underflows to exactly 0 in fp64


def _one(row, T=1.0):
    return sampler.denoise_sample(np.asarray(row, np.float64)[None, :], T, [3], [0], 1)


@pytest.mark.parametrize("V,expect", [(1024, 6.931471805599453), (262144, 12.476649250079015),
                                      (151936, 11.931214658529285)])
def test_uniform_row_entropy_is_log_v(V, expect):
    o = _one(np.full(V, 0.37))
    assert o.entropy[0] == pytest.approx(expect, abs=1e-12)
    assert expect == pytest.approx(math.log(V), abs=1e-12)
    assert o.argmax[0] == 0            # all tied -> lowest index


def test_one_hot_entropy_zero():
    row = np.full(1000, NEG)
    row[417] = 2.5
    o = _one(row)
    assert o.entropy[0] == 0.0
    assert o.argmax[0] == 417 and o.sample[0] == 417


@pytest.mark.parametrize("a,b", [(0.0, 0.0), (1.3, -0.2), (5.0, 0.0), (-3.0, 4.0)])
def test_two_point_entropy(a, b):
    row = np.full(64, NEG)
    row[5], row[40] = a, b
    p = 1.0 / (1.0 + math.exp(b - a))
    expect = -(p * math.log(p) + (1 - p) * math.log(1 - p))
    assert _one(row).entropy[0] == pytest.approx(expect, abs=1e-12)


@pytest.mark.parametrize("k", [1, 2, 3, 7, 256])
def test_k_equal_maxima_entropy_log_k(k):
    row = np.full(4096, NEG)
    idx = np.random.default_rng(k).choice(4096, k, replace=False)
    row[idx] = 1.25
    o = _one(row)
    assert o.entropy[0] == pytest.approx(math.log(k), abs=1e-12)
    assert o.argmax[0] == idx.min()


def test_entropy_matches_definition_and_shift_invariance():
    rng = np.random.default_rng(0)
    for T in (1.0, 0.7, 2.0):
        row = rng.normal(0, 3, 5000)
        p = sampler.probabilities(row, T)
        assert np.sum(p) == pytest.approx(1.0, abs=1e-12)
        o1 = _one(row, T)
        o2 = _one(row + 123.0, T)
        assert o1.entropy[0] == pytest.approx(sampler.entropy_direct(p), abs=1e-10)
        assert o2.entropy[0] == pytest.approx(o1.entropy[0], abs=1e-9)
        assert o1.row_lnz[0] == pytest.approx(np.log(np.sum(np.exp(row / T - np.max(row / T)))), abs=1e-12)
        assert o1.row_max[0] == np.max(row) / T


def test_argmax_is_first_occurrence_like_numpy():
    rng = np.random.default_rng(1)
    for _ in range(50):
        row = rng.integers(-3, 3, 300).astype(np.float64)   # many exact ties
        assert _one(row).argmax[0] == int(np.argmax(row))


def test_gumbel_max_follows_softmax():
    """One block (V <= 16): the flat Gumbel-max law."""
    V, n = 8, 20000
    logits = np.array([0.0, 1.0, -1.0, 2.0, 0.5, -2.0, 1.5, 0.0])
    rows = np.tile(logits, (n, 1))
    o = sampler.denoise_sample(rows, 1.0, [2024], [11], n)      # one request, n positions
    counts = np.bincount(o.sample, minlength=V)
    p = sampler.probabilities(logits, 1.0)
    assert stats.chisquare(counts, p * n).pvalue > 1e-4
    # temperature sharpens
    o2 = sampler.denoise_sample(rows, 0.25, [2024], [11], n)
    assert np.bincount(o2.sample, minlength=V)[3] > counts[3]


def test_single_block_is_flat_gumbel_max():
    """A row of at most 16 ids is one block: the two-level draw is the flat draw, id for id."""
    rng = np.random.default_rng(7)
    for V in (1, 5, 12, 16):
        x = rng.normal(0, 2, V)
        for pos in range(20):
            cand, _ = sampler.gumbel_candidate(x, 99, pos, 4)
            assert cand == sampler.flat_gumbel_candidate(x, 99, pos, 4)[0]


def _rank_buckets(p: np.ndarray, n: int, n_tail: int = 12, cell: float = 25.0):
    """Chi-square cells for n draws from p: every id expected >= `cell` times on its own (the top
    ids), the rest in order of decreasing probability cut into about `n_tail` buckets of equal mass.
    Returns (cell of each id, expected count per cell)."""
    order = np.argsort(-p, kind="stable")
    cells = np.empty(p.size, np.int64)
    top = int(np.sum(p[order] * n >= cell))
    cells[order[:top]] = np.arange(top)
    rest = order[top:]
    cum = np.cumsum(p[rest]) / max(np.sum(p[rest]), 1e-300)
    cells[rest] = top + np.minimum((cum * n_tail).astype(np.int64), n_tail - 1)
    expect = np.bincount(cells, weights=p, minlength=top + n_tail) * n
    return cells, expect


def _chi2_pvalue(cells, expect, draws):
    obs = np.bincount(cells[np.asarray(draws)], minlength=expect.size)
    keep = expect > 0
    return stats.chisquare(obs[keep], expect[keep] * obs.sum() / expect[keep].sum()).pvalue


def test_flat_draw_follows_softmax():
    """The Gumbel-max theorem for the flat draw, on a Zipf row of 4096 ids over 4000 positions."""
    x = synth.bf16_bits_to_f32(synth.zipf_logits_bf16(0, "flat-law", 1, 4096)[0]).astype(np.float64)
    n = 4000
    draws = [sampler.flat_gumbel_candidate(x, 5, pos, 2)[0] for pos in range(n)]
    cells, expect = _rank_buckets(sampler.probabilities(x, 1.0), n)
    assert _chi2_pvalue(cells, expect, draws) > 1e-4


def test_two_level_and_flat_draws_have_one_law():
    """Both draws on one row of 2048 ids (128 blocks), 4000 positions each: a two-sample
    chi-square test over probability-rank cells finds no difference, and each follows softmax."""
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1.5, 2048)
    x[rng.choice(2048, 6, replace=False)] += 4.0
    n = 4000
    lm = sampler.block_log_mass(x)
    two = [sampler.gumbel_candidate(x, 8, pos, 3, log_mass=lm)[0] for pos in range(n)]
    flat = [sampler.flat_gumbel_candidate(x, 8, pos, 3)[0] for pos in range(n)]
    cells, expect = _rank_buckets(sampler.probabilities(x, 1.0), n)
    table = np.stack([np.bincount(cells[two], minlength=expect.size),
                      np.bincount(cells[flat], minlength=expect.size)])
    table = table[:, table.sum(axis=0) > 0]
    assert stats.chi2_contingency(table).pvalue > 1e-4
    assert _chi2_pvalue(cells, expect, two) > 1e-4 and _chi2_pvalue(cells, expect, flat) > 1e-4


@pytest.mark.parametrize("kind", ["peaked", "diffuse"])
def test_two_level_law_at_full_vocabulary(kind):
    """V = 262144 on the benchmark's Zipf rows: of 16 generated rows, the lowest-entropy one (a few
    ids carry most of the mass) and the highest (mass spread over the whole vocabulary).  Over
    3000 positions the candidates follow softmax(x) -- the top ids one by one, the rest in
    equal-mass probability-rank buckets -- and their blocks follow the block masses Z_b / Z."""
    V, n = 262144, 3000
    rows = synth.bf16_bits_to_f32(synth.zipf_logits_bf16(0, "law-262144", 16, V)).astype(np.float64)
    H = [sampler.softmax_stats(r)[3] for r in rows]
    x = rows[int(np.argmin(H) if kind == "peaked" else np.argmax(H))]
    lm = sampler.block_log_mass(x)
    draws = np.array([sampler.gumbel_candidate(x, 21, pos, 6, log_mass=lm)[0] for pos in range(n)])
    p = sampler.probabilities(x, 1.0)
    cells, expect = _rank_buckets(p, n)
    assert _chi2_pvalue(cells, expect, draws) > 1e-4
    pb = p.reshape(-1, 16).sum(axis=1)
    bcells, bexpect = _rank_buckets(pb, n)
    assert _chi2_pvalue(bcells, bexpect, draws // 16) > 1e-4
    if kind == "peaked":
        assert expect.size > 13          # several ids are cells of their own
    else:
        assert np.max(p) * n < 25        # no id reaches a cell of its own: all mass in rank buckets


def test_two_level_draw_follows_softmax_across_blocks():
    """Three blocks with a short last one (16 + 16 + 8 ids): the candidate law is softmax(x)."""
    V, n = 40, 20000
    logits = np.random.default_rng(8).normal(0, 1.0, V)
    logits[3] += 2.0
    logits[35] += 2.5                                   # mass in the short block too
    rows = np.tile(logits, (n, 1))
    o = sampler.denoise_sample(rows, 1.0, [77], [5], n)
    counts = np.bincount(o.sample, minlength=V)
    p = sampler.probabilities(logits, 1.0)
    keep = p * n >= 5                                   # chi-square cells with enough expectation
    obs, exp = counts[keep], p[keep] * n
    if not keep.all():
        obs, exp = np.append(obs, counts[~keep].sum()), np.append(exp, p[~keep].sum() * n)
    assert stats.chisquare(obs, exp).pvalue > 1e-4


def test_winning_block_law_is_block_mass():
    """64 blocks of a ramp: the block of the candidate is drawn with probability Z_b / Z."""
    V, n = 1024, 6000
    logits = np.linspace(-1.5, 1.5, V)
    rows = np.tile(logits, (n, 1))
    o = sampler.denoise_sample(rows, 1.0, [3], [9], n)
    blocks = np.bincount(o.sample // 16, minlength=64)
    pb = sampler.probabilities(logits, 1.0).reshape(64, 16).sum(axis=1)
    assert stats.chisquare(blocks, pb * n).pvalue > 1e-4


def test_block_noise_map_is_a_bijection():
    from oracle import philox
    b = np.arange(1 << 14)
    c0, w = philox.block_counter_word(b)
    assert len(set(zip(c0.tolist(), w.tolist()))) == b.size
    assert np.all((w >= 0) & (w < 4))
    # blocks p, p + 128, p + 256, p + 384 of each run of 512 share one counter, words 0..3
    for S in (0, 3):
        for p in (0, 77, 127):
            bb = 512 * S + p + 128 * np.arange(4)
            cc, ww = philox.block_counter_word(bb)
            assert np.all(cc == cc[0]) and np.array_equal(ww, np.arange(4))


def test_samples_depend_on_seed_step_position_only():
    rng = np.random.default_rng(2)
    rows = rng.normal(0, 1, (6, 500))
    a = sampler.denoise_sample(rows, 1.0, [5, 6], [10, 10], 3)
    b = sampler.denoise_sample(rows, 1.0, [5, 6], [10, 10], 3)
    c = sampler.denoise_sample(rows, 1.0, [5, 6], [11, 10], 3)
    assert np.array_equal(a.sample, b.sample)
    assert not np.array_equal(a.sample[:3], c.sample[:3])      # diffuse rows: a new step redraws
    assert np.array_equal(a.sample[3:], c.sample[3:])


def test_argmax_only_and_inactive():
    rows = np.random.default_rng(3).normal(0, 1, (4, 100))
    o = sampler.denoise_sample(rows, 1.0, [1, 2], [0, 0], 2, argmax_only=True, active=[1, 0])
    assert np.array_equal(o.argmax[:2], np.argmax(rows[:2], axis=1))
    assert np.all(o.argmax[2:] == -1) and np.all(o.sample == -1)
