"""Per-position denoise sampler: softmax statistics, entropy, argmax, Gumbel-max candidate.

Follows the DiffusionGemma/vLLM page (discuss.pytorch.kr, "DiffusionGemma: the
first dLLM natively supported by vLLM"):
  * section "Entropy-based denoising": every position is resampled each step
    and its confidence is the entropy H(p) = -sum_i p_i log p_i of its
    predicted distribution;
  * section "DiffusionGemmaModelState and DiffusionSampler", denoise case:
    logits are divided by the temperature T and a candidate is drawn with the
    Gumbel-max trick; the argmax canvas is recorded.

Readings (the pages are silent): natural log (nats); H clamped at 0; argmax
and sample ties go to the lowest vocabulary index; the Gumbel noise is the
Philox streams of ``oracle.philox``.  Also returned: m = max_i x_i and
ln Z = ln sum_i exp(x_i - m), which define p_i = exp(x_i - m - ln Z) for the
self-conditioning step.

Two forms of the Gumbel-max candidate:
  * ``flat_gumbel_candidate`` is the trick as the page states it: one Gumbel
    value g_i per vocabulary id and the candidate argmax_i (x_i + g_i).  Its law
    is softmax(x) (the Gumbel-max theorem).
  * ``gumbel_candidate`` is the draw the step computes (a reading of the page,
    which fixes no noise layout): two levels over blocks of 16 consecutive
    ids (the last block of a row may be shorter).  Block b has log-mass
    L_b = ln sum_{i in b} exp(x_i) and its own noise G_b; the winning block is
    b* = argmax_b (L_b + G_b); inside b* the candidate is argmax_{i in b*}
    (x_i + g_i) with per-id noise.  The maximum of Gumbel-perturbed values over
    a set is Gumbel with the set's log-mass as location, independent of which
    element attains it, so b* is drawn with probability Z_b / Z and the
    candidate with probability exp(x_i) / Z: the flat draw's law, with one
    noise value per 16 ids at the first level.  The per-id noise g_i is the
    flat draw's own, so a row of at most 16 ids (one block) gives exactly the
    flat candidate.

Pinned by tests/test_oracle_sampler.py: entropy closed forms (uniform row ->
ln V, one-hot -> 0, two-point, k equal maxima -> ln k), shift invariance,
sum p = 1, argmax == numpy.argmax, chi-square tests that the flat candidate
follows softmax(x), that the two-level candidate follows softmax(x) and its
block the block masses (up to V = 262144 on peaked and diffuse Zipf rows),
that both draws give the same law, and that one block reduces to the flat draw.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import philox


@dataclass
class SampleOut:
    entropy: np.ndarray     # float64 [rows]
    argmax: np.ndarray      # int64 [rows]
    sample: np.ndarray      # int64 [rows]  (-1 when argmax-only)
    row_max: np.ndarray     # float64 [rows]  m = max x
    row_lnz: np.ndarray     # float64 [rows]  ln sum exp(x - m)
    argmax_gap: np.ndarray  # float64 [rows]  top value minus best value at any other index
    key_gap: np.ndarray     # float64 [rows]  same for the Gumbel keys (inf when argmax-only)


def softmax_stats(x: np.ndarray):
    """m, Z, S and H for one row of scaled logits x (fp64).

    m = max x;  Z = sum exp(x - m);  S = sum exp(x - m) (x - m);
    H = -sum p log p with p = exp(x - m) / Z, which expands to ln Z - S / Z.
    """
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x)
    e = np.exp(x - m)
    Z = np.sum(e)
    S = np.sum(e * (x - m))
    H = max(0.0, float(np.log(Z) - S / Z))
    return float(m), float(Z), float(S), H


def entropy_direct(p: np.ndarray) -> float:
    """-sum p log p with 0 log 0 = 0 (the definition, used by the pins)."""
    p = np.asarray(p, dtype=np.float64)
    nz = p > 0
    return float(-np.sum(p[nz] * np.log(p[nz])))


def _top2_gap(v: np.ndarray) -> float:
    if v.size < 2:
        return np.inf
    i = int(np.argmax(v))
    rest = np.delete(v, i)
    return float(v[i] - np.max(rest))


def flat_gumbel_candidate(x: np.ndarray, seed: int, pos: int, step: int):
    """The Gumbel-max trick as stated: argmax_i (x_i + g_i), one Gumbel value per id.

    g_i is the per-id noise of ``philox.inner_gumbels`` (stream GUMBEL_INNER).  Returns
    (candidate id, top-2 gap of the keys).
    """
    x = np.asarray(x, dtype=np.float64)
    key = x + philox.inner_gumbels(seed, pos, step, 0, x.size)
    return int(np.argmax(key)), _top2_gap(key)


def block_log_mass(x: np.ndarray) -> np.ndarray:
    """L_b = ln sum_{i in b} exp(x_i) over blocks of 16 consecutive ids (the last may be shorter)."""
    x = np.asarray(x, dtype=np.float64)
    V = x.size
    nb = (V + philox.GUMBEL_BLOCK - 1) // philox.GUMBEL_BLOCK
    xb = np.full(nb * philox.GUMBEL_BLOCK, -np.inf)
    xb[:V] = x
    xb = xb.reshape(nb, philox.GUMBEL_BLOCK)
    mb = np.max(xb, axis=1)
    return mb + np.log(np.sum(np.exp(xb - mb[:, None]), axis=1))


def gumbel_candidate(x: np.ndarray, seed: int, pos: int, step: int, log_mass=None):
    """Two-level Gumbel-max candidate for one row of scaled logits x (fp64).

    log_mass: ``block_log_mass(x)`` when the caller already has it (draws over many positions
    of one row).  Returns (candidate id, key gap): the gap is the smaller of the top-2 gaps of
    the block keys and of the keys inside the winning block (near-tie accounting).
    """
    x = np.asarray(x, dtype=np.float64)
    V = x.size
    if log_mass is None:
        log_mass = block_log_mass(x)
    bkey = log_mass + philox.block_gumbels(seed, pos, step, log_mass.size)
    b = int(np.argmax(bkey))
    lo, hi = b * philox.GUMBEL_BLOCK, min((b + 1) * philox.GUMBEL_BLOCK, V)
    ikey = x[lo:hi] + philox.inner_gumbels(seed, pos, step, lo, hi)
    return lo + int(np.argmax(ikey)), min(_top2_gap(bkey), _top2_gap(ikey))


def denoise_sample(logits: np.ndarray, temperature: float, seeds, steps, rows_per_req: int,
                   argmax_only: bool = False, active=None, draw: str = "two_level") -> SampleOut:
    """Sampler over logit rows.

    draw: "two_level" (the step's draw, ``gumbel_candidate``) or "flat" (``flat_gumbel_candidate``).

    logits: [rows, V] (already decoded to float; bf16 inputs are exact in fp64).
    Row r belongs to request r // rows_per_req at canvas position r % rows_per_req;
    seeds[req] (uint64) and steps[req] key its Gumbel noise.
    active: optional per-request flags; rows of inactive requests are left as NaN / -1.
    """
    logits = np.asarray(logits)
    rows, V = logits.shape
    out = SampleOut(*(np.full(rows, np.nan) for _ in range(1)),
                    argmax=np.full(rows, -1, np.int64), sample=np.full(rows, -1, np.int64),
                    row_max=np.full(rows, np.nan), row_lnz=np.full(rows, np.nan),
                    argmax_gap=np.full(rows, np.inf), key_gap=np.full(rows, np.inf))
    for r in range(rows):
        req, pos = divmod(r, rows_per_req)
        if active is not None and not active[req]:
            continue
        l = logits[r].astype(np.float64)
        out.argmax[r] = int(np.argmax(l))          # first occurrence = lowest index
        out.argmax_gap[r] = _top2_gap(l)
        if argmax_only:
            continue
        x = l / float(temperature)
        m, Z, _S, H = softmax_stats(x)
        out.entropy[r] = H
        out.row_max[r] = m
        out.row_lnz[r] = np.log(Z)
        cand = flat_gumbel_candidate if draw == "flat" else gumbel_candidate
        out.sample[r], out.key_gap[r] = cand(x, int(seeds[req]), pos, int(steps[req]))
    return out


def probabilities(logits_row: np.ndarray, temperature: float) -> np.ndarray:
    x = np.asarray(logits_row, dtype=np.float64) / float(temperature)
    e = np.exp(x - np.max(x))
    return e / np.sum(e)
