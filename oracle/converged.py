"""Convergence test, commit and block restart.

Follows the DiffusionGemma/vLLM page:
  * section "Entropy-based denoising": a canvas has converged when its argmax
    prediction has stopped changing for several consecutive steps AND its mean
    per-token entropy is below a confidence threshold; a step cap stops the
    loop otherwise; what is committed is the clean argmax canvas, not the
    noisy sampled canvas;
  * section "DiffusionGemmaModelState and DiffusionSampler": three cases --
    prefill (random canvas, nothing emitted), denoise, commit (emit the argmax
    canvas, report C sampled tokens, re-initialise the canvas and the
    per-request state); denoise steps report zero sampled tokens.

Readings: "unchanged for k steps" = k consecutive whole-canvas equalities
with the previous step's argmax (the first step of a block has no previous);
the mean is over all C positions of the current step, compared strictly; the
cap commits the final argmax too; a restart draws the new canvas from the
Philox INIT stream at the request's global step and turns self-conditioning
off; the global step advances on every call.  A request whose step_in_block
is negative is in the prefill case: it receives a random canvas and starts
its first block (no convergence test, nothing emitted).

Pinned by tests/test_oracle_converged.py (hand-built histories with known
outcomes: constant argmax at zero entropy commits after k+1 steps, an
alternating argmax runs to the cap, a mean exactly at the threshold does not
converge, prefill/restart tokens equal the Philox INIT stream).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import philox


@dataclass
class LoopState:
    """Per-request diffusion state (all arrays indexed by request)."""
    canvas: np.ndarray          # int64 [B, C]
    prev_argmax: np.ndarray     # int64 [B, C]
    unchanged: np.ndarray       # int64 [B]
    step_in_block: np.ndarray   # int64 [B]
    step_global: np.ndarray     # int64 [B]
    sc_on: np.ndarray           # uint8 [B]

    def copy(self):
        return LoopState(*(np.array(getattr(self, f), copy=True) for f in
                           ("canvas", "prev_argmax", "unchanged", "step_in_block", "step_global", "sc_on")))


@dataclass
class ConvergedOut:
    committed: np.ndarray    # uint8 [B]
    out_tokens: np.ndarray   # int64 [B, C] (valid where committed)
    steps_used: np.ndarray   # int64 [B]   (valid where committed)
    num_sampled: np.ndarray  # int64 [B]
    mean_gap: np.ndarray     # float64 [B]  |mean H - tau| (near-tie measure)
    extra: dict = field(default_factory=dict)


def converged(argmax: np.ndarray, entropy: np.ndarray, state: LoopState, k: int, tau: float,
              max_steps: int, seeds, V: int, active=None) -> ConvergedOut:
    """Advance `state` in place by one step and report commits."""
    argmax = np.asarray(argmax, dtype=np.int64)
    entropy = np.asarray(entropy, dtype=np.float64)
    B, C = state.canvas.shape
    committed = np.zeros(B, np.uint8)
    out_tokens = np.zeros((B, C), np.int64)
    steps_used = np.zeros(B, np.int64)
    num_sampled = np.zeros(B, np.int64)
    mean_gap = np.full(B, np.inf)
    for b in range(B):
        if active is not None and not active[b]:
            continue
        g = int(state.step_global[b])
        if state.step_in_block[b] < 0:          # prefill case: random canvas, first block begins
            state.canvas[b] = philox.random_tokens(int(seeds[b]), g, np.arange(C), V, philox.INIT)
            state.unchanged[b] = 0
            state.step_in_block[b] = 0
            state.sc_on[b] = 0
            state.step_global[b] = g + 1
            continue
        same = state.step_in_block[b] > 0 and bool(np.all(argmax[b] == state.prev_argmax[b]))
        state.unchanged[b] = state.unchanged[b] + 1 if same else 0
        mean_h = float(np.sum(entropy[b])) / C
        mean_gap[b] = abs(mean_h - tau)
        conv = state.unchanged[b] >= k and mean_h < tau
        cap = state.step_in_block[b] + 1 >= max_steps
        if conv or cap:
            committed[b] = 1
            out_tokens[b] = argmax[b]
            steps_used[b] = state.step_in_block[b] + 1
            num_sampled[b] = C
            state.canvas[b] = philox.random_tokens(int(seeds[b]), g, np.arange(C), V, philox.INIT)
            state.unchanged[b] = 0
            state.step_in_block[b] = 0
            state.sc_on[b] = 0
        else:
            state.step_in_block[b] += 1
            state.sc_on[b] = 1
        state.prev_argmax[b] = argmax[b]
        state.step_global[b] = g + 1
    return ConvergedOut(committed=committed, out_tokens=out_tokens, steps_used=steps_used,
                        num_sampled=num_sampled, mean_gap=mean_gap)
