"""Mixed-mask canvas attention over a paged KV prefix.

Follows:
  * DiffusionGemma/vLLM page, section "Two modes, one set of weights": the
    encoder mode (prompt prefill and the commit pass) is causal and writes
    K/V to the cache; the decoder (denoise) mode is bidirectional over the
    canvas and only reads the cache;
  * same page, section "Dynamic per-sequence causal attention": requests at
    different phases share one batch, causality is a per-request property,
    and in the three-request figure a canvas of 4 sees its whole context and
    every canvas key while prefill/commit rows see keys up to themselves;
  * single-pass-reads page ("DiffusionGemma's execution path merged",
    portfolio.ywsung.com), section on keeping each row's visibility: a merged
    launch splits a request into input (causal) rows and canvas rows that
    share the request's KV block table; in the p0 p1 c0 c1 example p0 sees
    p0, p1 sees p0 p1, and c0, c1 see p0 p1 c0 c1;
  * DiffusionGemma/vLLM page, section on symmetric sliding-window attention:
    in a sliding-window layer of window W a causal row keeps the one-sided
    window (itself and the W keys before it) while a canvas row sees W keys on
    each side of itself (2W + 1 keys), so a canvas only sees the context
    tokens that fall inside its window; only the right edge differs between
    the two kinds of request.

Visibility rule for one request with ``cached`` prefix tokens, ``n_causal``
causal rows and ``n_canvas`` canvas rows (key index space: cache positions
0 .. cached + n_causal - 1, then the canvas rows; row and key positions are
their indices in that space, so causal row j sits at cached + j and canvas row
j at cached + n_causal + j):
  causal row at position p -> keys 0 .. p
  canvas row               -> every key of the request
With a window W > 0 the visible set is further cut to positions
[p - W, p] for a causal row and [p - W, p + W] for a canvas row.  W = 0 means
a full-attention layer (no window).  Reading: the page counts the window in
tokens of the request's sequence; the positions above are that sequence's
positions (the cached prefix, the causal rows, then the canvas).
Causal rows' K/V are appended to the paged cache at positions cached + j
before any row reads; canvas K/V are never written.  Scores use
scale * q . k, softmax over visible keys only, output = sum p v.  GQA: query
head h reads KV head h // (Hq / Hkv).  No position encoding is applied (the
inputs are synthetic Q/K/V).

E4M3 paged cache (canvas_attention_e4m3; DiffusionGemma/vLLM page, section "Quantized checkpoint
support", the FP8 model): the cache holds OCP E4M3 codes, a cached key or value is
scale * decode(code) (one scale for K, one for V); the causal rows of a launch are quantised when
appended (code = encode(x / scale), round to nearest even, saturating); within the launch every
key at a position >= cached, causal or canvas, is used at input precision (the rows are this
launch's own activations), and the cache is read only below `cached`.  Reading: the page names
FP8 weights and fully dynamic activations without fixing where the cache quantises; keeping the
launch's own rows unquantised follows the canvas rows, which never enter the cache.

Pinned by tests/test_oracle_attention.py: the p0/p1/c0/c1 and the
three-request visibility fixtures in tests/golden/ (with and without the
W = 2 window), brute-force dense-mask attention on random shapes (window
decided by a position predicate there), one-visible-key and equal-score special cases,
and permutation / page-relabelling invariances.
"""
from __future__ import annotations

import numpy as np


def visibility_mask(cached: int, n_causal: int, n_canvas: int, window: int = 0) -> np.ndarray:
    """Boolean [n_causal + n_canvas, cached + n_causal + n_canvas] mask of one request."""
    nk = cached + n_causal + n_canvas
    rows = n_causal + n_canvas
    mask = np.zeros((rows, nk), dtype=bool)
    for j in range(n_causal):
        p = cached + j
        lo = max(0, p - window) if window > 0 else 0
        mask[j, lo:p + 1] = True
    for j in range(n_canvas):
        p = cached + n_causal + j
        if window > 0:
            mask[n_causal + j, max(0, p - window):min(nk, p + window + 1)] = True
        else:
            mask[n_causal + j, :] = True
    return mask


def dense_mask_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, scale: float) -> np.ndarray:
    """Brute force: q [R, D], k/v [K, D], mask [R, K] -> out [R, D] (fp64).  Rows with no visible key give 0."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    out = np.zeros((q.shape[0], v.shape[1]))
    for r in range(q.shape[0]):
        idx = np.nonzero(mask[r])[0]
        if idx.size == 0:
            continue
        s = scale * (k[idx] @ q[r])
        w = np.exp(s - np.max(s))
        out[r] = (w / np.sum(w)) @ v[idx]
    return out


def append_causal_kv(k_cache, v_cache, k_new, v_new, page_table, row0, cached, n_causal, page0, page_size):
    """Write one request's causal-row K/V ([rows, Hkv, D]) into its pages at positions cached + j."""
    for j in range(n_causal):
        pos = cached + j
        page = int(page_table[page0 + pos // page_size])
        k_cache[page, :, pos % page_size, :] = k_new[row0 + j]
        v_cache[page, :, pos % page_size, :] = v_new[row0 + j]


def gather_request_kv(k_cache, v_cache, k_new, v_new, page_table, row0, cached, n_causal, n_canvas, page0, page_size):
    """Keys/values of one request in key-index order: cache positions, then canvas rows. [nk, Hkv, D]."""
    n_cache = cached + n_causal
    Hkv, D = k_cache.shape[1], k_cache.shape[3]
    K = np.zeros((n_cache + n_canvas, Hkv, D), dtype=np.float64)
    Vv = np.zeros_like(K)
    for pos in range(n_cache):
        page = int(page_table[page0 + pos // page_size])
        K[pos] = k_cache[page, :, pos % page_size, :]
        Vv[pos] = v_cache[page, :, pos % page_size, :]
    c0 = row0 + n_causal
    K[n_cache:] = k_new[c0:c0 + n_canvas]
    Vv[n_cache:] = v_new[c0:c0 + n_canvas]
    return K, Vv


def canvas_attention(q, k, v, k_cache, v_cache, page_table, splits, page_size: int, scale: float):
    """Oracle for one launch.

    q [rows, Hq, D]; k, v [rows, Hkv, D]; caches [pages, Hkv, page_size, D] (float arrays);
    splits: iterable of (row0, cached, n_causal, n_canvas, page0[, window]); window 0 (or absent)
    is full attention.
    Returns (out [rows, Hq, D] fp64, k_cache', v_cache' with causal K/V appended).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    rows, Hq, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    out = np.zeros((rows, Hq, D))
    splits = [tuple(int(t) for t in s) + (0,) * (6 - len(s)) for s in splits]
    for (row0, cached, n_causal, n_canvas, page0, _w) in splits:
        append_causal_kv(kc, vc, k, v, page_table, row0, cached, n_causal, page0, page_size)
    for (row0, cached, n_causal, n_canvas, page0, window) in splits:
        K, Vv = gather_request_kv(kc, vc, k, v, page_table, row0, cached, n_causal, n_canvas, page0, page_size)
        mask = visibility_mask(cached, n_causal, n_canvas, window)
        nr = n_causal + n_canvas
        for h in range(Hq):
            hk = h // group
            out[row0:row0 + nr, h] = dense_mask_attention(q[row0:row0 + nr, h], K[:, hk], Vv[:, hk], mask, scale)
    return out, kc, vc


def canvas_attention_e4m3(q, k, v, kc8, vc8, k_scale: float, v_scale: float, page_table, splits, page_size: int,
                          scale: float):
    """Oracle for one launch over an E4M3 paged cache.

    q [rows, Hq, D]; k, v [rows, Hkv, D] (float arrays); kc8, vc8 [pages, Hkv, page_size, D] uint8 codes;
    splits as in canvas_attention.  Returns (out [rows, Hq, D] fp64, kc8', vc8' with the causal rows'
    codes appended).
    """
    from . import fp8
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    kc8_new = np.array(kc8, dtype=np.uint8, copy=True)
    vc8_new = np.array(vc8, dtype=np.uint8, copy=True)
    kc = fp8.decode_table(kc8, k_scale)          # the cache as it was before this launch's appends
    vc = fp8.decode_table(vc8, v_scale)
    rows, Hq, D = q.shape
    group = Hq // k.shape[1]
    out = np.zeros((rows, Hq, D))
    splits = [tuple(int(t) for t in s) + (0,) * (6 - len(s)) for s in splits]
    for (row0, cached, n_causal, n_canvas, page0, window) in splits:
        for j in range(n_causal):
            pos = cached + j
            page = int(page_table[page0 + pos // page_size])
            kc8_new[page, :, pos % page_size, :] = fp8.encode_e4m3(k[row0 + j] / k_scale)
            vc8_new[page, :, pos % page_size, :] = fp8.encode_e4m3(v[row0 + j] / v_scale)
    for (row0, cached, n_causal, n_canvas, page0, window) in splits:
        nr = n_causal + n_canvas
        K = np.zeros((cached + nr, k.shape[1], D))
        Vv = np.zeros_like(K)
        for pos in range(cached):
            page = int(page_table[page0 + pos // page_size])
            K[pos] = kc[page, :, pos % page_size, :]
            Vv[pos] = vc[page, :, pos % page_size, :]
        K[cached:] = k[row0:row0 + nr]
        Vv[cached:] = v[row0:row0 + nr]
        mask = visibility_mask(cached, n_causal, n_canvas, window)
        for h in range(Hq):
            hk = h // group
            out[row0:row0 + nr, h] = dense_mask_attention(q[row0:row0 + nr, h], K[:, hk], Vv[:, hk], mask, scale)
    return out, kc8_new, vc8_new
