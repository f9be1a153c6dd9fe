"""Self-conditioning: probability-weighted token embedding + small gated MLP.

Follows the DiffusionGemma/vLLM page:
  * section "Self-conditioning": between steps the model is conditioned on its
    own previous prediction -- the previous step's full softmax is turned into
    a probability-weighted mean of the token embeddings, passed through a
    small gated MLP and added to the canvas embedding of the next pass; the
    feedback is zero in the encoder passes (prefill, commit);
  * section "DiffusionGemmaModelState and DiffusionSampler": prepare_inputs()
    embeds the canvas tokens and applies this self-conditioning from the
    per-request state.

Computation per canvas row r (fp64):
  p_r = exp(x_r - m_r - ln Z_r)             (this step's softmax, from the sampler's m, ln Z)
  s_r = p_r . E                              (E: [V, d] token embeddings)
  y_r = (gelu_tanh(s_r W_gate) * (s_r W_up)) W_down
  x_next_r = E[canvas_r] + (y_r if self-conditioning is on for the request else 0)

Readings: the gated MLP is bias-free GeGLU with the tanh form of GELU (the
Gemma family's convention); no sqrt(d) embedding scale; x_next is rounded to
bf16 (nearest even) when the table is bf16.

Pinned by tests/test_oracle_selfcond.py: one-hot p gives the embedding row
exactly, uniform p gives the column mean of E, s matches a numpy fp64
matmul, MLP(0) = 0, gelu_tanh matches torch's tanh-approximate GELU
(an independent library routine) and the self-conditioning-off path is the
plain embedding lookup.
"""
from __future__ import annotations

import numpy as np


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, np.float64)
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def probs_from_stats(logits: np.ndarray, temperature: float, row_max: np.ndarray, row_lnz: np.ndarray) -> np.ndarray:
    x = np.asarray(logits, np.float64) / float(temperature)
    return np.exp(x - np.asarray(row_max, np.float64)[:, None] - np.asarray(row_lnz, np.float64)[:, None])


def prob_embed(P: np.ndarray, E: np.ndarray) -> np.ndarray:
    """s = P . E in fp64."""
    return np.asarray(P, np.float64) @ np.asarray(E, np.float64)


def gated_mlp(s: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    s = np.asarray(s, np.float64)
    g = s @ np.asarray(w_gate, np.float64)
    u = s @ np.asarray(w_up, np.float64)
    return (gelu_tanh(g) * u) @ np.asarray(w_down, np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (ties to even), returned as fp64."""
    # via fp32: a value within half an fp32 ulp of a bf16 halfway point may round differently
    # from a direct fp64 -> bf16 rounding; outputs are compared normwise, so this is immaterial.
    f = np.asarray(x, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def selfcond_embed(P: np.ndarray, canvas: np.ndarray, sc_on: np.ndarray, E: np.ndarray,
                   w_gate, w_up, w_down, rows_per_req: int, to_bf16: bool):
    """Returns (x_next [rows, d], s [rows, d], y [rows, d]) in fp64 (x_next rounded if to_bf16)."""
    E = np.asarray(E, np.float64)
    s = prob_embed(P, E)
    y = gated_mlp(s, w_gate, w_up, w_down)
    tok = np.asarray(canvas, np.int64).reshape(-1)
    on = np.repeat(np.asarray(sc_on, bool), rows_per_req)
    x = E[tok] + np.where(on[:, None], y, 0.0)
    if to_bf16:
        x = round_bf16(x)
    return x, s, y
