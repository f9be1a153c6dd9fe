"""Helpers shared by the GPU parity tests: uploads, tolerances and near-tie accounting.

Tolerances (stated once, used by every parity test):
  integers (argmax, sample, accept mask, tokens, steps): bit-exact, except near-ties,
      which are counted and reported: argmax or Gumbel-key top-2 gap < 1e-5, running
      entropy total within 1e-3 nats of the budget, |mean entropy - tau| < 1e-3;
  entropy: |delta| <= 1e-3 nats;  probabilities: relative 1e-3;
  P.E and the MLP / next-step embedding: per row ||delta|| / ||ref|| <= 1e-3;
  attention: |delta| <= 2e-2 (bf16) or 1e-4 (fp32).
"""
from __future__ import annotations

import numpy as np
import pytest

import synth

TIE_GAP = 1e-5
BUDGET_TIE = 1e-3
MEAN_TIE = 1e-3
TOL_ENTROPY = 1e-3
TOL_PROB_REL = 1e-3
TOL_NORM_REL = 1e-3
TOL_ATT_BF16 = 2e-2
TOL_ATT_F32 = 1e-4

NEAR_TIES: dict = {}


def report_tie(kind: str, n: int = 1):
    NEAR_TIES[kind] = NEAR_TIES.get(kind, 0) + n


def torch_mod():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def dev_bf16(a_u16: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a, dtype=None):
    torch = torch_mod()
    t = torch.as_tensor(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host_f64(t) -> np.ndarray:
    """Device tensor (bf16 / fp32 / ints) -> float64 numpy (bf16 decoded exactly)."""
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def rel_norm_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    got = np.asarray(got, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    return np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-300)


def check_sampler_rows(got: dict, ref, rows, argmax_only=False):
    """Compare GPU sampler outputs (host numpy dict) with the oracle on the listed rows."""
    bad = []
    for i, r in enumerate(rows):
        if got["argmax"][i] != ref.argmax[r]:
            if 0 < ref.argmax_gap[r] < TIE_GAP:      # exact ties must match (lowest index)
                report_tie("argmax_gap")
            else:
                bad.append(("argmax", r, got["argmax"][i], ref.argmax[r]))
        if argmax_only:
            continue
        if abs(got["entropy"][i] - ref.entropy[r]) > TOL_ENTROPY:
            bad.append(("entropy", r, got["entropy"][i], ref.entropy[r]))
        if got["sample"][i] != ref.sample[r]:
            if ref.key_gap[r] < TIE_GAP:
                report_tie("gumbel_key_gap")
            else:
                bad.append(("sample", r, got["sample"][i], ref.sample[r], ref.key_gap[r]))
        if abs(got["row_max"][i] - ref.row_max[r]) > 1e-6 * max(1.0, abs(ref.row_max[r])):
            bad.append(("row_max", r, got["row_max"][i], ref.row_max[r]))
        if abs(got["row_lnz"][i] - ref.row_lnz[r]) > 1e-4:
            bad.append(("row_lnz", r, got["row_lnz"][i], ref.row_lnz[r]))
    assert not bad, bad[:10]


def check_bf16_output(got: np.ndarray, exact: np.ndarray, pre_rel: float = 3 * TOL_NORM_REL):
    """A bf16 output against the oracle's unrounded fp64 value.

    A stored bf16 value cannot be closer than half a bf16 step (2^(e-7) in [2^e, 2^(e+1)));
    the check is that every element lies within one step of the exact value, widened by
    `pre_rel` times the row's rms (the fp16/fp32 path's own error before the final rounding,
    whose normwise size is checked separately at 1e-3 on the fp32 outputs), and that the
    row's normwise error stays within bf16's unit roundoff 2^-8.
    """
    got = np.asarray(got, np.float64)
    exact = np.asarray(exact, np.float64)
    mag = np.maximum(np.abs(exact), 1e-30)
    step = 2.0 ** (np.floor(np.log2(mag)) - 7)
    rms = np.sqrt(np.mean(exact ** 2, axis=-1, keepdims=True))
    err = np.abs(got - exact)
    assert np.all(err <= step + pre_rel * rms), float((err / (step + pre_rel * rms)).max())
    assert rel_norm_err(got, exact).max() <= 2.0 ** -8


def zipf_bf16(seed, tag, rows, V):
    return synth.zipf_logits_bf16(seed, tag, rows, V)


def sampler_oracle_row(row, seed, pos, step):
    """Oracle for one row at canvas position `pos` (a request of pos + 1 rows whose last row is this one)."""
    from oracle import sampler as _osamp
    x = np.asarray(row, np.float64)
    m, Z, S, H = _osamp.softmax_stats(x)
    cand, key_gap = _osamp.gumbel_candidate(x, seed, pos, step)
    srt = np.sort(x)
    return _osamp.SampleOut(entropy=np.array([H]), argmax=np.array([int(np.argmax(x))]),
                           sample=np.array([cand]), row_max=np.array([m]),
                           row_lnz=np.array([np.log(Z)]), argmax_gap=np.array([srt[-1] - srt[-2]]),
                           key_gap=np.array([key_gap]))


def oracle_pe_slabs(Pm: np.ndarray, table_rows, V: int, slab: int = 16384) -> np.ndarray:
    """s = P . E in fp64 by the oracle's prob_embed, summed over slabs of `slab` table rows so that
    the full 262144 x 4096 table never sits in host memory at once; table_rows(v0, v1) returns the
    fp64 rows v0 .. v1 - 1 of E."""
    from oracle import selfcond as _osc
    s = None
    for v0 in range(0, V, slab):
        v1 = min(V, v0 + slab)
        part = _osc.prob_embed(Pm[:, v0:v1], table_rows(v0, v1))
        s = part if s is None else s + part
    return s


def torch_table_rows(E):
    """table_rows for a device bf16 / fp32 table (exact fp64 copies of its rows)."""
    return lambda v0, v1: E[v0:v1].float().cpu().numpy().astype(np.float64)
