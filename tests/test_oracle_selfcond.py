"""Pins for oracle.selfcond: exact special cases and an independent library GELU."""
import numpy as np
import pytest
import torch

from oracle import selfcond, sampler


def test_one_hot_p_gives_embedding_row():
    rng = np.random.default_rng(0)
    E = rng.normal(0, 1 / 8, (300, 16))
    P = np.zeros((3, 300))
    P[0, 7] = P[1, 299] = P[2, 0] = 1.0
    np.testing.assert_array_equal(selfcond.prob_embed(P, E), E[[7, 299, 0]])


def test_uniform_p_gives_column_mean():
    E = np.random.default_rng(1).normal(0, 1, (1024, 8))
    P = np.full((1, 1024), 1 / 1024)
    np.testing.assert_allclose(selfcond.prob_embed(P, E)[0], E.mean(axis=0), atol=1e-14)


def test_probs_from_sampler_stats_are_softmax():
    rng = np.random.default_rng(2)
    L = rng.normal(0, 3, (4, 777))
    o = sampler.denoise_sample(L, 0.8, [1], [0], 4)
    P = selfcond.probs_from_stats(L, 0.8, o.row_max, o.row_lnz)
    for r in range(4):
        np.testing.assert_allclose(P[r], sampler.probabilities(L[r], 0.8), rtol=1e-12, atol=1e-300)


def test_gelu_tanh_matches_torch():
    z = np.linspace(-8, 8, 2001)
    ref = torch.nn.functional.gelu(torch.tensor(z, dtype=torch.float64), approximate="tanh").numpy()
    np.testing.assert_allclose(selfcond.gelu_tanh(z), ref, rtol=1e-14, atol=1e-15)
    assert selfcond.gelu_tanh(np.array([0.0]))[0] == 0.0


def test_mlp_zero_and_linearity_of_up_branch():
    rng = np.random.default_rng(3)
    wg, wu, wd = rng.normal(0, .02, (16, 32)), rng.normal(0, .02, (16, 32)), rng.normal(0, .02, (32, 16))
    assert np.all(selfcond.gated_mlp(np.zeros((2, 16)), wg, wu, wd) == 0)
    s = rng.normal(0, 1, (2, 16))
    # independent restatement with torch ops: down(gelu_tanh(gate(s)) * up(s))
    ts = torch.tensor(s)
    ref = (torch.nn.functional.gelu(ts @ torch.tensor(wg), approximate="tanh") * (ts @ torch.tensor(wu))) @ torch.tensor(wd)
    np.testing.assert_allclose(selfcond.gated_mlp(s, wg, wu, wd), ref.numpy(), rtol=1e-12)


def test_geglu_gate_up_down_order_hand_worked():
    """Which projection goes through the GELU, and the orientation of all three weights, from a
    hand-worked case.  Pre-activations of magnitude >= 10 saturate the tanh in fp64, so the GELU
    passes z >= 10 through unchanged and sends z <= -10 to 0 exactly:
      s = (1, 0): gate = (10, 10), up = (3, 5)  -> hidden (30, 50) -> y = 30 (1, 2) + 50 (4, 8) = (230, 460)
      s = (0, 1): gate = (-12, 11), up = (2, 9) -> hidden (0, 99)  -> y = 99 (4, 8) = (396, 792)
    Swapping gate and up, or transposing any of the three matrices, gives other values (e.g. a
    transposed W_gate: (30, 60) for the first row; a transposed W_down: (130, 520))."""
    wg = np.array([[10.0, 10.0], [-12.0, 11.0]])
    wu = np.array([[3.0, 5.0], [2.0, 9.0]])
    wd = np.array([[1.0, 2.0], [4.0, 8.0]])
    y = selfcond.gated_mlp(np.eye(2), wg, wu, wd)
    np.testing.assert_array_equal(y, [[230.0, 460.0], [396.0, 792.0]])
    for bad in (selfcond.gated_mlp(np.eye(2), wu, wg, wd), selfcond.gated_mlp(np.eye(2), wg.T, wu, wd),
                selfcond.gated_mlp(np.eye(2), wg, wu.T, wd), selfcond.gated_mlp(np.eye(2), wg, wu, wd.T)):
        assert np.abs(bad - y).max() > 1.0


def test_selfcond_off_is_plain_lookup_and_bf16_rounding():
    rng = np.random.default_rng(4)
    E = rng.normal(0, 1 / 8, (50, 8))
    P = rng.dirichlet(np.ones(50), size=4)
    w = [rng.normal(0, .02, sh) for sh in ((8, 16), (8, 16), (16, 8))]
    canvas = np.array([[3, 4], [5, 6]])
    x, s, y = selfcond.selfcond_embed(P, canvas, np.array([0, 1]), E, *w, rows_per_req=2, to_bf16=False)
    np.testing.assert_array_equal(x[:2], E[[3, 4]])
    np.testing.assert_allclose(x[2:], E[[5, 6]] + y[2:], atol=1e-15)
    xb, _, _ = selfcond.selfcond_embed(P, canvas, np.array([0, 1]), E, *w, rows_per_req=2, to_bf16=True)
    ref = torch.tensor(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(xb, ref)
