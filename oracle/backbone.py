"""The one-layer fp32 backbone of the tiny closed loop (fp64 here).

One layer used two ways, as on the DiffusionGemma/vLLM page, section "Two
modes, one set of weights": the encoder pass (prompt prefill, commit) is
causal and writes K/V; the decoder pass over the canvas is bidirectional and
reads K/V.  Layer: q, k, v = x Wq, x Wk, x Wv; h = x + Attn(q, k, v) Wo;
logits = scale * h E^T (tied embedding / LM head).  Readings: no
normalisation layer, no position encoding, no sqrt(d) embedding scale.

Pinned by tests/test_oracle_traces.py against the hand-worked traces of
tests/golden/backbone_trace.txt: uniform attention under zero scores, a 1:3
weighting from a score difference of ln 3, the residual, the causal prefill
and commit passes that append K/V, the canvas pass that sees every key and
writes none, the orientation of Wv and Wo, and the tied LM head h E^T.
"""
from __future__ import annotations

import numpy as np

from . import attention


def layer(x, w, k_cache, v_cache, page_table, split, Hq, Hkv, D, page_size):
    """x [rows, d] fp64 -> (h [rows, d], k_cache', v_cache').  split = (row0, cached, n_causal, n_canvas, page0)."""
    x = np.asarray(x, np.float64)
    rows = x.shape[0]
    q = (x @ w["wq"]).reshape(rows, Hq, D)
    k = (x @ w["wk"]).reshape(rows, Hkv, D)
    v = (x @ w["wv"]).reshape(rows, Hkv, D)
    o, kc, vc = attention.canvas_attention(q, k, v, k_cache, v_cache, page_table, [split], page_size,
                                           1.0 / np.sqrt(D))
    h = x + o.reshape(rows, Hq * D) @ np.asarray(w["wo"], np.float64)
    return h, kc, vc


def lm_head(h, E, scale):
    return float(scale) * (np.asarray(h, np.float64) @ np.asarray(E, np.float64).T)
