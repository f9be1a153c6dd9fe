"""Python binding of libdg (the denoise step's C ABI): argument marshalling only.

Every function here has the name of the C entry point it calls, takes torch
tensors that already live on the GPU (torch provides device memory and
streams), passes their raw pointers through ctypes and raises ``DGError`` on a
non-zero status.  No arithmetic of the step happens in Python.  If the
shared library has not been built the import of any entry point fails loudly:
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "DGError", "lib", "DG_F32", "DG_BF16", "DG_SAMPLE_ARGMAX_ONLY", "SPLIT_FIELDS",
    "dg_version", "dg_philox4x32_10", "dg_canvas_attention", "dg_canvas_attention_ws_bytes",
    "dg_denoise_sample", "dg_denoise_sample_ws_bytes", "dg_entropy_accept", "dg_converged",
    "dg_selfcond_prepared_bytes", "dg_selfcond_prepare", "dg_selfcond_ws_bytes", "dg_selfcond_embed",
    "dg_allowed_probs", "dg_verify_prefix", "dg_linear", "dg_gather_rows", "EXPORTED",
    "dg_selfcond_operand_bytes", "dg_denoise_sample_sc", "dg_selfcond_ws_bytes_sc", "dg_selfcond_embed_sc",
    "dg_deficit_admit", "dg_e4m3_decode", "dg_selfcond_prepared_bytes_e4m3", "dg_selfcond_prepare_e4m3",
    "dg_selfcond_embed_sc_e4m3", "dg_canvas_attention_e4m3", "dg_denoise_sample_noalloc",
    "dg_denoise_sample_noalloc_max_bytes", "dg_lmhead_ws_bytes", "dg_lmhead_operand_bytes",
    "dg_lmhead_denoise_sample", "dg_selfcond_embed_lm", "dg_lmhead_prepared_bytes", "dg_lmhead_prepare",
    "dg_lmhead_denoise_sample_traced", "dg_accept_converged",
]

DG_F32, DG_BF16 = 0, 1
DG_SAMPLE_ARGMAX_ONLY = 1
SPLIT_FIELDS = ("row0", "cached", "n_causal", "n_canvas", "page0", "window")

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdg.so")

_p, _i32, _i64, _u32, _f32, _f64, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                          ctypes.c_float, ctypes.c_double, ctypes.c_size_t)

# name -> (restype, argtypes): mirrors include/dg.h
_SIGS = {
    "dg_version": (_i32, []),
    "dg_status_str": (ctypes.c_char_p, [_i32]),
    "dg_philox4x32_10": (_i32, [_p, _p, _i64, _p, _p]),
    "dg_canvas_attention_ws_bytes": (_sz, [_i32] * 8),
    "dg_canvas_attention": (_i32, [_p, _p, _p, _p, _p, _i32, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                   _i32, _f32, _i32, _p, _p, _sz, _p]),
    "dg_canvas_attention_e4m3": (_i32, [_p, _p, _p, _p, _p, _f32, _f32, _i32, _p, _i32, _p, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _i32, _f32, _p, _p, _sz, _p]),
    "dg_denoise_sample_ws_bytes": (_sz, [_i32, _i32]),
    "dg_denoise_sample": (_i32, [_p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _f32, _u32, _p, _p, _p, _p, _p, _p,
                                 _sz, _p]),
    "dg_denoise_sample_noalloc_max_bytes": (_sz, []),
    "dg_denoise_sample_noalloc": (_i32, [_p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _f32, _u32, _p, _p, _p, _p, _p,
                                         _p]),
    "dg_entropy_accept": (_i32, [_p, _p, _i32, _i32, _i32, _f64, _p, _p, _p, _p, _p, _p, _p]),
    "dg_converged": (_i32, [_p, _p, _i32, _i32, _i32, _i32, _f64, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                            _p, _p]),
    "dg_accept_converged": (_i32, [_p, _p, _p, _i32, _i32, _i32, _f64, _i32, _f64, _i32, _p, _p, _p, _p, _p, _p, _p,
                                   _p, _p, _p, _p, _p, _p, _p, _p]),
    "dg_selfcond_prepared_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "dg_selfcond_prepare": (_i32, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _p, _sz, _p]),
    "dg_selfcond_ws_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "dg_selfcond_embed": (_i32, [_p, _i64, _i32, _f32, _p, _p, _p, _p, _i32, _i32, _p, _p, _p, _p, _p, _i32, _i32,
                                 _i32, _p, _p, _p, _p, _sz, _p]),
    "dg_selfcond_embed_traced": (_i32, [_p, _i64, _i32, _f32, _p, _p, _p, _p, _i32, _i32, _p, _p, _p, _p, _p, _i32,
                                        _i32, _i32, _p, _p, _p, _p, _sz, _p, _p, _p]),
    "dg_selfcond_operand_bytes": (_sz, [_i32, _i32]),
    "dg_denoise_sample_sc": (_i32, [_p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _f32, _p, _p, _p, _p, _p, _p, _sz,
                                    _p, _sz, _p]),
    "dg_selfcond_ws_bytes_sc": (_sz, [_i32, _i32, _i32, _i32]),
    "dg_selfcond_embed_sc": (_i32, [_p, _p, _p, _p, _p, _i32, _i32, _p, _p, _i32, _i32, _i32, _p, _p, _p, _p, _sz,
                                    _p, _p, _p]),
    "dg_lmhead_ws_bytes": (_sz, [_i32, _i32, _i32]),
    "dg_lmhead_operand_bytes": (_sz, [_i32, _i32]),
    "dg_lmhead_prepared_bytes": (_sz, [_i32, _i32]),
    "dg_lmhead_prepare": (_i32, [_p, _i32, _i32, _p, _sz, _p]),
    "dg_lmhead_denoise_sample": (_i32, [_p, _i64, _p, _i32, _i32, _i32, _f32, _i32, _p, _p, _p, _f32, _p, _p, _p, _p,
                                        _p, _p, _sz, _p, _sz, _p]),
    "dg_lmhead_denoise_sample_traced": (_i32, [_p, _i64, _p, _i32, _i32, _i32, _f32, _i32, _p, _p, _p, _f32, _p, _p,
                                               _p, _p, _p, _p, _sz, _p, _sz, _p, _p, _p]),
    "dg_selfcond_embed_lm": (_i32, [_p, _p, _p, _p, _p, _i32, _i32, _p, _p, _i32, _i32, _i32, _p, _p, _p, _p, _sz,
                                    _p, _p, _p]),
    "dg_allowed_probs": (_i32, [_p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _f32, _p, _p, _p]),
    "dg_verify_prefix": (_i32, [_p, _p, _i32, _i32, _p, _p]),
    "dg_deficit_admit": (_i32, [_i64, _i64, _p, _i32, _p, _p, _p]),
    "dg_e4m3_decode": (_i32, [_p, _i64, _f32, _p, _p, _p]),
    "dg_selfcond_prepared_bytes_e4m3": (_sz, [_i32, _i32, _i32]),
    "dg_selfcond_prepare_e4m3": (_i32, [_p, _p, _p, _p, _i32, _i32, _i32, _p, _sz, _p]),
    "dg_selfcond_embed_sc_e4m3": (_i32, [_p, _p, _p, _p, _p, _i32, _i32, _p, _f32, _p, _i32, _i32, _i32, _p, _p, _p,
                                         _p, _sz, _p, _p, _p]),
    "dg_linear": (_i32, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _f32, _p]),
    "dg_gather_rows": (_i32, [_p, _i32, _i32, _i32, _p, _i32, _p, _p]),
}
EXPORTED = tuple(_SIGS)


class DGError(RuntimeError):
    pass


_LIB = None


def lib():
    """Load libdg.so (built in-tree by ``python -m denoise_step_amd.build``)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise DGError(f"{LIB_PATH} is missing; build it with `python -m denoise_step_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int, name: str):
    if status != 0:
        msg = lib().dg_status_str(status).decode()
        raise DGError(f"{name} failed with status {status} ({msg})")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise DGError("tensor arguments must live on the GPU")
    if not t.is_contiguous():
        raise DGError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    if t.dtype == torch.bfloat16:
        return DG_BF16
    if t.dtype == torch.float32:
        return DG_F32
    raise DGError(f"unsupported tensor dtype {t.dtype}")


def _ws(nbytes: int, ws, device):
    if nbytes == 0:
        return ws
    if ws is None or ws.numel() * ws.element_size() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def dg_version() -> int:
    return int(lib().dg_version())


def dg_philox4x32_10(ctr: torch.Tensor, key: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """ctr [n,4] int32/uint32 bits, key [n,2] -> out [n,4] (int32 storage of uint32 bits)."""
    n = ctr.shape[0]
    out = torch.empty((n, 4), dtype=torch.int32, device=ctr.device) if out is None else out
    _check(lib().dg_philox4x32_10(_ptr(ctr), _ptr(key), n, _ptr(out), _stream(stream)), "dg_philox4x32_10")
    return out


def dg_canvas_attention_ws_bytes(n_req, rows, max_rows, max_keys, Hq, Hkv, D, dtype) -> int:
    return int(lib().dg_canvas_attention_ws_bytes(n_req, rows, max_rows, max_keys, Hq, Hkv, D, dtype))


def dg_canvas_attention(q, k, v, k_cache, v_cache, page_table, splits, max_rows_per_req, max_keys_per_req,
                        scale, out=None, ws=None, stream=None):
    """q [rows,Hq,D], k/v [rows,Hkv,D], caches [pages,Hkv,page,D], page_table int32, splits int32 [n_req,6]."""
    rows, Hq, D = q.shape
    Hkv = k.shape[1]
    n_pages, _, page_size, _ = k_cache.shape
    n_req = splits.shape[0]
    dt = _dtype_code(q)
    out = torch.empty_like(q) if out is None else out
    nb = dg_canvas_attention_ws_bytes(n_req, rows, max_rows_per_req, max_keys_per_req, Hq, Hkv, D, dt)
    ws = _ws(nb, ws, q.device)
    _check(lib().dg_canvas_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), n_pages,
                                     _ptr(page_table), page_table.numel(), _ptr(splits), n_req, rows,
                                     max_rows_per_req, max_keys_per_req, Hq, Hkv, D, page_size, float(scale), dt,
                                     _ptr(out), _ptr(ws) if nb else None, nb, _stream(stream)),
           "dg_canvas_attention")
    return out


def dg_canvas_attention_e4m3(q, k, v, k_cache8, v_cache8, k_scale, v_scale, page_table, splits, max_rows_per_req,
                             max_keys_per_req, scale, out=None, ws=None, stream=None):
    """dg_canvas_attention over an E4M3 paged cache: k_cache8 / v_cache8 uint8 codes [pages, Hkv, page, D],
    values k_scale * code / v_scale * code (powers of two); q, k, v bf16."""
    rows, Hq, D = q.shape
    Hkv = k.shape[1]
    n_pages, _, page_size, _ = k_cache8.shape
    n_req = splits.shape[0]
    out = torch.empty_like(q) if out is None else out
    nb = dg_canvas_attention_ws_bytes(n_req, rows, max_rows_per_req, max_keys_per_req, Hq, Hkv, D, DG_BF16)
    ws = _ws(nb, ws, q.device)
    _check(lib().dg_canvas_attention_e4m3(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cache8), _ptr(v_cache8), float(k_scale),
                                          float(v_scale), n_pages, _ptr(page_table), page_table.numel(), _ptr(splits),
                                          n_req, rows, max_rows_per_req, max_keys_per_req, Hq, Hkv, D, page_size,
                                          float(scale), _ptr(out), _ptr(ws) if nb else None, nb, _stream(stream)),
           "dg_canvas_attention_e4m3")
    return out


def dg_denoise_sample_ws_bytes(rows, V) -> int:
    return int(lib().dg_denoise_sample_ws_bytes(rows, V))


def dg_denoise_sample(logits, V, rows_per_req, seed, step, temperature=1.0, active=None, argmax_only=False,
                      out=None, ws=None, stream=None):
    """logits [rows, ld] -> dict(entropy, argmax, sample, row_max, row_lnz) device tensors."""
    rows, ld = logits.shape
    dev = logits.device
    if out is None:
        out = dict(argmax=torch.empty(rows, dtype=torch.int32, device=dev))
        if not argmax_only:
            out.update(entropy=torch.empty(rows, dtype=torch.float32, device=dev),
                       sample=torch.empty(rows, dtype=torch.int32, device=dev),
                       row_max=torch.empty(rows, dtype=torch.float32, device=dev),
                       row_lnz=torch.empty(rows, dtype=torch.float32, device=dev))
    nb = dg_denoise_sample_ws_bytes(rows, V)
    ws = _ws(nb, ws, dev)
    g = out.get
    _check(lib().dg_denoise_sample(_ptr(logits), ld, _dtype_code(logits), rows, V, rows_per_req, _ptr(seed),
                                   _ptr(step), _ptr(active), float(temperature),
                                   DG_SAMPLE_ARGMAX_ONLY if argmax_only else 0, _ptr(g("entropy")),
                                   _ptr(g("argmax")), _ptr(g("sample")), _ptr(g("row_max")), _ptr(g("row_lnz")),
                                   _ptr(ws), nb, _stream(stream)), "dg_denoise_sample")
    return out


def dg_denoise_sample_noalloc_max_bytes() -> int:
    return int(lib().dg_denoise_sample_noalloc_max_bytes())


def dg_denoise_sample_noalloc(logits, V, rows_per_req, seed, step, out, temperature=1.0, active=None,
                              argmax_only=False, stream=None):
    """dg_denoise_sample without a workspace (the library's fixed per-device scratch); `out` holds the
    caller's preallocated output tensors (argmax, and entropy / sample / row_max / row_lnz unless
    argmax_only), so the call allocates nothing."""
    rows, ld = logits.shape
    g = out.get
    _check(lib().dg_denoise_sample_noalloc(_ptr(logits), ld, _dtype_code(logits), rows, V, rows_per_req, _ptr(seed),
                                           _ptr(step), _ptr(active), float(temperature),
                                           DG_SAMPLE_ARGMAX_ONLY if argmax_only else 0, _ptr(g("entropy")),
                                           _ptr(g("argmax")), _ptr(g("sample")), _ptr(g("row_max")),
                                           _ptr(g("row_lnz")), _stream(stream)), "dg_denoise_sample_noalloc")
    return out


def dg_selfcond_operand_bytes(rows, V) -> int:
    return int(lib().dg_selfcond_operand_bytes(rows, V))


def dg_denoise_sample_sc(logits, V, rows_per_req, seed, step, temperature=1.0, active=None, out=None, ws=None,
                         sc_operand=None, stream=None):
    """dg_denoise_sample that also writes the self-conditioning operand; returns (outputs, operand)."""
    rows, ld = logits.shape
    dev = logits.device
    if out is None:
        out = dict(argmax=torch.empty(rows, dtype=torch.int32, device=dev),
                   entropy=torch.empty(rows, dtype=torch.float32, device=dev),
                   sample=torch.empty(rows, dtype=torch.int32, device=dev),
                   row_max=torch.empty(rows, dtype=torch.float32, device=dev),
                   row_lnz=torch.empty(rows, dtype=torch.float32, device=dev))
    nb = dg_denoise_sample_ws_bytes(rows, V)
    ws = _ws(nb, ws, dev)
    ob = dg_selfcond_operand_bytes(rows, V)
    sc_operand = _ws(ob, sc_operand, dev)
    g = out.get
    _check(lib().dg_denoise_sample_sc(_ptr(logits), ld, _dtype_code(logits), rows, V, rows_per_req, _ptr(seed),
                                      _ptr(step), _ptr(active), float(temperature), _ptr(g("entropy")),
                                      _ptr(g("argmax")), _ptr(g("sample")), _ptr(g("row_max")), _ptr(g("row_lnz")),
                                      _ptr(ws), nb, _ptr(sc_operand), ob, _stream(stream)), "dg_denoise_sample_sc")
    return out, sc_operand


def dg_entropy_accept(entropy, sample, canvas, V, budget, seed, step, active=None, accept=None, n_accept=None,
                      stream=None):
    B, C = canvas.shape
    _check(lib().dg_entropy_accept(_ptr(entropy), _ptr(sample), B, C, V, float(budget), _ptr(seed), _ptr(step),
                                   _ptr(active), _ptr(canvas), _ptr(accept), _ptr(n_accept), _stream(stream)),
           "dg_entropy_accept")


def dg_converged(argmax, entropy, V, k, tau, max_steps, seed, state: dict, active=None, stream=None):
    """state: dict of device tensors prev_argmax, unchanged, step_in_block, step_global, canvas, sc_on,
    committed, out_tokens, steps_used, num_sampled (updated in place)."""
    B, C = state["canvas"].shape
    s = state
    _check(lib().dg_converged(_ptr(argmax), _ptr(entropy), B, C, V, int(k), float(tau), int(max_steps), _ptr(seed),
                              _ptr(active), _ptr(s["prev_argmax"]), _ptr(s["unchanged"]), _ptr(s["step_in_block"]),
                              _ptr(s["step_global"]), _ptr(s["canvas"]), _ptr(s["sc_on"]), _ptr(s["committed"]),
                              _ptr(s["out_tokens"]), _ptr(s["steps_used"]), _ptr(s["num_sampled"]),
                              _stream(stream)), "dg_converged")


def dg_accept_converged(entropy, sample, argmax, V, budget, k, tau, max_steps, seed, state: dict, active=None,
                        accept=None, n_accept=None, stream=None):
    """dg_entropy_accept then dg_converged in one launch (prefill case: dg_converged only); state as in
    dg_converged (updated in place, canvas included)."""
    B, C = state["canvas"].shape
    s = state
    _check(lib().dg_accept_converged(_ptr(entropy), _ptr(sample), _ptr(argmax), B, C, V, float(budget), int(k),
                                     float(tau), int(max_steps), _ptr(seed), _ptr(active), _ptr(s["prev_argmax"]),
                                     _ptr(s["unchanged"]), _ptr(s["step_in_block"]), _ptr(s["step_global"]),
                                     _ptr(s["canvas"]), _ptr(s["sc_on"]), _ptr(s["committed"]), _ptr(s["out_tokens"]),
                                     _ptr(s["steps_used"]), _ptr(s["num_sampled"]), _ptr(accept), _ptr(n_accept),
                                     _stream(stream)), "dg_accept_converged")


def dg_selfcond_prepared_bytes(V, d, hidden, dtype) -> int:
    return int(lib().dg_selfcond_prepared_bytes(V, d, hidden, dtype))


def dg_selfcond_prepare(E, w_gate, w_up, w_down, stream=None):
    """Build the fp16 operand copies used by the bf16 path (E^T, [W_gate|W_up]^T, W_down^T)."""
    V, d = E.shape
    hidden = w_gate.shape[1]
    dt = _dtype_code(E)
    nb = dg_selfcond_prepared_bytes(V, d, hidden, dt)
    prepared = torch.empty(max(nb, 1), dtype=torch.uint8, device=E.device)
    _check(lib().dg_selfcond_prepare(_ptr(E), _ptr(w_gate), _ptr(w_up), _ptr(w_down), V, d, hidden, dt,
                                     _ptr(prepared), nb, _stream(stream)), "dg_selfcond_prepare")
    return prepared


def dg_selfcond_ws_bytes(rows, V, d, hidden, dtype) -> int:
    return int(lib().dg_selfcond_ws_bytes(rows, V, d, hidden, dtype))


def dg_selfcond_embed(logits, V, row_max, row_lnz, sc_on, canvas, E, w_gate, w_up, w_down, prepared,
                      temperature=1.0, x_out=None, s_out=None, y_out=None, ws=None, stream=None, pe_events=None):
    """pe_events: optional (start, stop) pair of raw hipEvent_t handles (ints) recorded around the P.E kernel."""
    B, C = canvas.shape
    rows, ld = logits.shape
    d = E.shape[1]
    hidden = w_gate.shape[1]
    dt = _dtype_code(logits)
    x_out = torch.empty((rows, d), dtype=E.dtype, device=E.device) if x_out is None else x_out
    nb = dg_selfcond_ws_bytes(rows, V, d, hidden, dt)
    ws = _ws(nb, ws, logits.device)
    ev0, ev1 = (None, None) if pe_events is None else (int(pe_events[0]), int(pe_events[1]))
    _check(lib().dg_selfcond_embed_traced(_ptr(logits), ld, dt, float(temperature), _ptr(row_max), _ptr(row_lnz),
                                          _ptr(sc_on), _ptr(canvas), B, C, _ptr(E), _ptr(w_gate), _ptr(w_up),
                                          _ptr(w_down), _ptr(prepared), V, d, hidden, _ptr(x_out), _ptr(s_out),
                                          _ptr(y_out), _ptr(ws), nb, ev0, ev1, _stream(stream)),
           "dg_selfcond_embed_traced")
    return x_out


def dg_selfcond_ws_bytes_sc(rows, V, d, hidden) -> int:
    return int(lib().dg_selfcond_ws_bytes_sc(rows, V, d, hidden))


def dg_selfcond_embed_sc(sc_operand, V, row_max, row_lnz, sc_on, canvas, E, prepared, hidden, x_out=None,
                         s_out=None, y_out=None, ws=None, stream=None, pe_events=None):
    """dg_selfcond_embed on the operand written by dg_denoise_sample_sc."""
    B, C = canvas.shape
    rows = B * C
    d = E.shape[1]
    x_out = torch.empty((rows, d), dtype=E.dtype, device=E.device) if x_out is None else x_out
    nb = dg_selfcond_ws_bytes_sc(rows, V, d, hidden)
    ws = _ws(nb, ws, E.device)
    ev0, ev1 = (None, None) if pe_events is None else (int(pe_events[0]), int(pe_events[1]))
    _check(lib().dg_selfcond_embed_sc(_ptr(sc_operand), _ptr(row_max), _ptr(row_lnz), _ptr(sc_on), _ptr(canvas), B,
                                      C, _ptr(E), _ptr(prepared), V, d, hidden, _ptr(x_out), _ptr(s_out),
                                      _ptr(y_out), _ptr(ws), nb, ev0, ev1, _stream(stream)), "dg_selfcond_embed_sc")
    return x_out


def dg_lmhead_ws_bytes(rows, V, d) -> int:
    return int(lib().dg_lmhead_ws_bytes(rows, V, d))


def dg_lmhead_operand_bytes(rows, V) -> int:
    return int(lib().dg_lmhead_operand_bytes(rows, V))


def dg_lmhead_prepared_bytes(V, d) -> int:
    return int(lib().dg_lmhead_prepared_bytes(V, d))


def dg_lmhead_prepare(E, prepared=None, stream=None):
    """The table E [V][d] bf16 re-laid for dg_lmhead_denoise_sample (uint8 device buffer)."""
    V, d = E.shape
    nb = dg_lmhead_prepared_bytes(V, d)
    prepared = _ws(nb, prepared, E.device)
    _check(lib().dg_lmhead_prepare(_ptr(E), V, d, _ptr(prepared), nb, _stream(stream)), "dg_lmhead_prepare")
    return prepared


def dg_lmhead_denoise_sample(h, prepared, V, scale, rows_per_req, seed, step, temperature=1.0, active=None, out=None,
                             ws=None, operand=None, stream=None, events=None):
    """The LM head logits = scale h E^T fused with the sampler (h [rows][d] bf16, prepared from
    dg_lmhead_prepare); returns (outputs, operand) with the operand for dg_selfcond_embed_lm.
    events: optional (start, stop) hipEvent_t handles recorded around the fused LM-head kernel."""
    rows, ldh = h.shape
    d = ldh
    dev = h.device
    if out is None:
        out = dict(argmax=torch.empty(rows, dtype=torch.int32, device=dev),
                   entropy=torch.empty(rows, dtype=torch.float32, device=dev),
                   sample=torch.empty(rows, dtype=torch.int32, device=dev),
                   row_max=torch.empty(rows, dtype=torch.float32, device=dev),
                   row_lnz=torch.empty(rows, dtype=torch.float32, device=dev))
    nb = dg_lmhead_ws_bytes(rows, V, d)
    ws = _ws(nb, ws, dev)
    ob = dg_lmhead_operand_bytes(rows, V)
    operand = _ws(ob, operand, dev)
    g = out.get
    ev0, ev1 = (None, None) if events is None else (int(events[0]), int(events[1]))
    _check(lib().dg_lmhead_denoise_sample_traced(_ptr(h), ldh, _ptr(prepared), rows, V, d, float(scale), rows_per_req,
                                                 _ptr(seed), _ptr(step), _ptr(active), float(temperature),
                                                 _ptr(g("entropy")), _ptr(g("argmax")), _ptr(g("sample")),
                                                 _ptr(g("row_max")), _ptr(g("row_lnz")), _ptr(ws), nb, _ptr(operand),
                                                 ob, ev0, ev1, _stream(stream)), "dg_lmhead_denoise_sample_traced")
    return out, operand


def dg_selfcond_embed_lm(lm_operand, V, row_max, row_lnz, sc_on, canvas, E, prepared, hidden, x_out=None,
                         s_out=None, y_out=None, ws=None, stream=None, pe_events=None):
    """dg_selfcond_embed on the operand written by dg_lmhead_denoise_sample."""
    B, C = canvas.shape
    rows = B * C
    d = E.shape[1]
    x_out = torch.empty((rows, d), dtype=E.dtype, device=E.device) if x_out is None else x_out
    nb = dg_selfcond_ws_bytes_sc(rows, V, d, hidden)
    ws = _ws(nb, ws, E.device)
    ev0, ev1 = (None, None) if pe_events is None else (int(pe_events[0]), int(pe_events[1]))
    _check(lib().dg_selfcond_embed_lm(_ptr(lm_operand), _ptr(row_max), _ptr(row_lnz), _ptr(sc_on), _ptr(canvas), B,
                                      C, _ptr(E), _ptr(prepared), V, d, hidden, _ptr(x_out), _ptr(s_out),
                                      _ptr(y_out), _ptr(ws), nb, ev0, ev1, _stream(stream)), "dg_selfcond_embed_lm")
    return x_out


def dg_e4m3_decode(codes, scale=1.0, out16=None, stream=None):
    """uint8 E4M3 codes (numel % 8 == 0) -> float32 values times scale (and fp16 values into out16)."""
    out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _check(lib().dg_e4m3_decode(_ptr(codes), codes.numel(), float(scale), _ptr(out), _ptr(out16), _stream(stream)),
           "dg_e4m3_decode")
    return out


def dg_selfcond_prepared_bytes_e4m3(V, d, hidden) -> int:
    return int(lib().dg_selfcond_prepared_bytes_e4m3(V, d, hidden))


def dg_selfcond_prepare_e4m3(E8, w_gate, w_up, w_down, stream=None):
    """E8: uint8 E4M3 codes [V, d]; MLP weights bf16.  Builds the E4M3 E^T and the fp16 MLP operands."""
    V, d = E8.shape
    hidden = w_gate.shape[1]
    nb = dg_selfcond_prepared_bytes_e4m3(V, d, hidden)
    prepared = torch.empty(max(nb, 1), dtype=torch.uint8, device=E8.device)
    _check(lib().dg_selfcond_prepare_e4m3(_ptr(E8), _ptr(w_gate), _ptr(w_up), _ptr(w_down), V, d, hidden,
                                          _ptr(prepared), nb, _stream(stream)), "dg_selfcond_prepare_e4m3")
    return prepared


def dg_selfcond_embed_sc_e4m3(sc_operand, V, row_max, row_lnz, sc_on, canvas, E8, e_scale, prepared, hidden,
                              x_out=None, s_out=None, y_out=None, ws=None, stream=None, pe_events=None):
    """dg_selfcond_embed_sc against an E4M3 table (values e_scale * decode(E8)); x_out is bf16."""
    B, C = canvas.shape
    rows = B * C
    d = E8.shape[1]
    x_out = torch.empty((rows, d), dtype=torch.bfloat16, device=E8.device) if x_out is None else x_out
    nb = dg_selfcond_ws_bytes_sc(rows, V, d, hidden)
    ws = _ws(nb, ws, E8.device)
    ev0, ev1 = (None, None) if pe_events is None else (int(pe_events[0]), int(pe_events[1]))
    _check(lib().dg_selfcond_embed_sc_e4m3(_ptr(sc_operand), _ptr(row_max), _ptr(row_lnz), _ptr(sc_on),
                                           _ptr(canvas), B, C, _ptr(E8), float(e_scale), _ptr(prepared), V, d, hidden,
                                           _ptr(x_out), _ptr(s_out), _ptr(y_out), _ptr(ws), nb, ev0, ev1,
                                           _stream(stream)), "dg_selfcond_embed_sc_e4m3")
    return x_out


def dg_allowed_probs(logits, V, slot_row, offsets, ids, temperature=1.0, q=None, answer=None, stream=None):
    n_rows, ld = logits.shape
    n_slots = slot_row.numel()
    q = torch.empty(ids.numel(), dtype=torch.float32, device=logits.device) if q is None else q
    answer = torch.empty(n_slots, dtype=torch.int32, device=logits.device) if answer is None else answer
    _check(lib().dg_allowed_probs(_ptr(logits), ld, _dtype_code(logits), n_rows, n_slots, V, _ptr(slot_row),
                                  _ptr(offsets), _ptr(ids), float(temperature), _ptr(q), _ptr(answer),
                                  _stream(stream)), "dg_allowed_probs")
    return q, answer


def dg_verify_prefix(draft, target, accepted=None, stream=None):
    B, L = draft.shape
    accepted = torch.empty(B, dtype=torch.int32, device=draft.device) if accepted is None else accepted
    _check(lib().dg_verify_prefix(_ptr(draft), _ptr(target), B, L, _ptr(accepted), _stream(stream)),
           "dg_verify_prefix")
    return accepted


def dg_deficit_admit(budget, decode_tokens, queue, deficit):
    """Host call: queue = prefill token counts in arrival order.  Returns (n_admitted, deficit, tokens)."""
    n_q = len(queue)
    arr = (ctypes.c_int64 * max(n_q, 1))(*[int(x) for x in queue])
    d = ctypes.c_int64(int(deficit))
    n = ctypes.c_int32(0)
    tok = ctypes.c_int64(0)
    _check(lib().dg_deficit_admit(int(budget), int(decode_tokens), ctypes.cast(arr, _p), n_q, ctypes.byref(d),
                                  ctypes.byref(n), ctypes.byref(tok)), "dg_deficit_admit")
    return n.value, d.value, tok.value


def dg_linear(A, B, residual=None, trans_b=False, alpha=1.0, out=None, stream=None):
    M, K = A.shape
    N = B.shape[0] if trans_b else B.shape[1]
    out = torch.empty((M, N), dtype=torch.float32, device=A.device) if out is None else out
    _check(lib().dg_linear(_ptr(A), _ptr(B), _ptr(residual), _ptr(out), M, N, K, int(bool(trans_b)), float(alpha),
                           _stream(stream)), "dg_linear")
    return out


def dg_gather_rows(table, idx, out=None, stream=None):
    n_table, d = table.shape
    n = idx.numel()
    out = torch.empty((n, d), dtype=table.dtype, device=table.device) if out is None else out
    _check(lib().dg_gather_rows(_ptr(table), n_table, d, _dtype_code(table), _ptr(idx), n, _ptr(out),
                                _stream(stream)), "dg_gather_rows")
    return out
