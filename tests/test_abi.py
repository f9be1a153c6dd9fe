"""CPU checks of the boundary: libdg loads, exports every entry point of include/dg.h, and rejects bad
arguments on the host before launching anything (no GPU needed for these calls)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "dg.h")).read()
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    import denoise_step_amd as dg
    if not os.path.exists(dg.LIB_PATH):
        from denoise_step_amd import build
        build.build()
    return dg.lib()


def test_every_declared_symbol_is_exported(L):
    names = header_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(L, n), n
    import denoise_step_amd as dg
    assert set(names) == set(dg.EXPORTED)


def test_version_and_status_strings(L):
    assert L.dg_version() >= 100
    assert L.dg_status_str(0) == b"ok"
    assert L.dg_status_str(-3).startswith(b"workspace")


def test_host_validation_rejects_before_launch(L):
    # null logits / bad sizes / unsupported dtype / misaligned ld / missing workspace
    args = dict(logits=None, ld=1024, dtype=1, rows=16, V=1024, rpr=16)
    f = lambda **kw: L.dg_denoise_sample(kw.get("logits", 16), kw.get("ld", 1024), kw.get("dtype", 1),
                                         kw.get("rows", 16), kw.get("V", 1024), kw.get("rpr", 16), 64, 64, None,
                                         kw.get("T", 1.0), 0, 64, 64, 64, 64, 64, kw.get("ws", 64),
                                         kw.get("wsb", 1 << 20), None)
    assert f(logits=None) == -1
    assert f(rows=0) == -1
    assert f(rows=15) == -1                    # rows not a multiple of rows_per_req
    assert f(ld=1000) == -1                    # ld < V
    assert f(dtype=7) == -2
    assert f(ld=1028) == -2                    # ld % 8 != 0
    assert f(logits=17) == -2                  # not 16-byte aligned
    assert f(T=0.0) == -1
    assert f(ws=None) == -3
    assert f(wsb=1) == -3
    assert L.dg_entropy_accept(64, 64, 1, 1025, 10, 1.0, 64, 64, None, 64, None, None, None) == -1
    assert L.dg_converged(64, 64, 1, 0, 10, 2, 0.5, 32, 64, None, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, None) == -1
    # attention: unsupported head_dim / page size, Hq % Hkv
    att = lambda D=128, ps=16, Hq=16, Hkv=8: L.dg_canvas_attention(64, 64, 64, 64, 64, 4, 64, 4, 64, 1, 16, 16, 32,
                                                                     Hq, Hkv, D, ps, 0.1, 1, 64, None, 0, None)
    assert att(D=96) == -2 and att(ps=32) == -2 and att(Hq=12, Hkv=8) == -1
    # the MFMA path's longest key span: 261120 keys pass validation (then the missing workspace is
    # reported), one more is unsupported
    keys = lambda mk: L.dg_canvas_attention(64, 64, 64, 64, 64, 4, 64, 4, 64, 1, 16, 16, mk, 16, 8, 128, 16, 0.1, 1,
                                            64, None, 0, None)
    assert keys(261120) == -3 and keys(261121) == -2
    # self-conditioning: bf16 requires d, hidden multiples of 128 and a prepared table
    assert L.dg_selfcond_embed(64, 1024, 1, 1.0, 64, 64, 64, 64, 1, 16, 64, 64, 64, 64, None, 1024, 128, 128, 64,
                               None, None, 64, 1 << 30, None) == -1
    assert L.dg_selfcond_embed(64, 1024, 1, 1.0, 64, 64, 64, 64, 1, 16, 64, 64, 64, 64, 64, 1024, 96, 128, 64,
                               None, None, 64, 1 << 30, None) == -2
    assert L.dg_selfcond_embed(64, 1024, 1, 1.0, 64, 64, 64, 64, 1, 16, 64, 64, 64, 64, 64, 1024, 8320, 128, 64,
                               None, None, 64, 1 << 30, None) == -2      # d above 8192


def test_fused_operand_entry_points_validate(L):
    sc = lambda dtype=1, op=64, opb=1 << 30: L.dg_denoise_sample_sc(64, 1024, dtype, 16, 1024, 16, 64, 64, None, 1.0,
                                                                     64, 64, 64, 64, 64, 64, 1 << 20, op, opb, None)
    assert sc(dtype=0) == -2                     # the operand path reads bf16 logits only
    assert sc(op=None) == -1
    assert sc(opb=1) == -3
    assert L.dg_selfcond_operand_bytes(256, 262144) >= 256 * 262144 * 2 + 256 * 16 * 4
    emb = lambda op=64, d=128, wsb=1 << 30: L.dg_selfcond_embed_sc(op, 64, 64, 64, 64, 1, 16, 64, 64, 1024, d, 128,
                                                                   64, None, None, 64, wsb, None, None, None)
    assert emb(op=None) == -1
    assert emb(d=96) == -2
    assert emb(wsb=1) == -3
    assert L.dg_selfcond_ws_bytes_sc(256, 262144, 4096, 1024) > 0


def test_lmhead_entry_points_validate(L):
    # h, ldh, E, rows, V, d, scale, rows_per_req, seed, step, active, T, 5 outputs, ws, ws_bytes, operand, bytes, stream
    call = lambda V=16384, d=256, scale=1.0, rows=32, rpr=16, ldh=256, wsb=1 << 30, opb=1 << 30, h=64: \
        L.dg_lmhead_denoise_sample(h, ldh, 64, rows, V, d, scale, rpr, 64, 64, None, 1.0, 64, 64, 64, 64, 64, 64,
                                   wsb, 64, opb, None)
    assert call(h=None) == -1
    assert call(V=16392) == -2                   # V % 16 != 0
    assert call(d=200, ldh=200) == -2            # d % 128 != 0
    assert call(scale=0.0) == -1
    assert call(scale=float("inf")) == -1
    assert call(rpr=5) == -1                     # rows % rows_per_req != 0
    assert call(ldh=128) == -1                   # ldh < d
    assert call(ldh=260) == -2                   # ldh % 8 != 0
    assert call(wsb=1) == -3
    assert call(opb=1) == -3
    assert L.dg_lmhead_ws_bytes(256, 262144, 4096) >= 256 * 4096 * 2 + 256 * 1024 * 32
    assert L.dg_lmhead_operand_bytes(256, 262144) >= L.dg_selfcond_operand_bytes(256, 262144) + 256 * 4
    assert L.dg_lmhead_prepared_bytes(262144, 4096) == 262144 * 4096 * 2
    prep = lambda V=16384, d=256, nb=1 << 30, E=64: L.dg_lmhead_prepare(E, V, d, 64, nb, None)
    assert prep(E=None) == -1
    assert prep(V=100) == -2
    assert prep(d=96) == -2
    assert prep(nb=16) == -3
    emb = lambda op=64, V=1024, wsb=1 << 30: L.dg_selfcond_embed_lm(op, 64, 64, 64, 64, 1, 16, 64, 64, V, 128, 128,
                                                                    64, None, None, 64, wsb, None, None, None)
    assert emb(op=None) == -1
    assert emb(V=1000) == -2
    assert emb(wsb=1) == -3


def test_workspace_sizes(L):
    assert L.dg_denoise_sample_ws_bytes(256, 262144) == 256 * 4 * 32      # 4 chunks of 65536 logits per row
    assert L.dg_selfcond_ws_bytes(256, 262144, 4096, 1024, 1) >= 256 * 262144 * 2
    assert L.dg_selfcond_prepared_bytes(262144, 4096, 1024, 1) >= 262144 * 4096 * 2 + 3 * 4096 * 1024 * 2


def test_e4m3_attention_validates(L):
    import ctypes
    import denoise_step_amd as dg
    p = ctypes.c_void_p(16)
    sp = ctypes.c_void_p(32)
    f = L.dg_canvas_attention_e4m3
    # non power-of-two scale, unsupported head dim, bad sizes: rejected before any launch
    args = lambda ks, D, nreq: (p, p, p, p, p, ks, 0.5, 4, p, 4, sp, nreq, 8, 8, 8, 2, 1, D, 16, 0.1, p, None, 0, None)
    assert f(*args(0.3, 128, 1)) == -2
    assert f(*args(0.25, 64, 1)) == -2
    assert f(*args(0.25, 128, 0)) == -1


def test_noalloc_sampler_rejects_sizes_beyond_its_scratch(L):
    """The allocation-free sampler checks its fixed scratch on the host before anything else: a
    launch needing more chunk partials than the array holds returns DG_E_SCRATCH (-5) and launches
    nothing (V = 2^20 is 16 chunks of 65536 ids per row; 16385 rows need 262160 > 262144)."""
    assert L.dg_denoise_sample_noalloc_max_bytes() == 8 << 20
    assert L.dg_denoise_sample_ws_bytes(16385, 1 << 20) > L.dg_denoise_sample_noalloc_max_bytes()
    call = lambda rows, V: L.dg_denoise_sample_noalloc(64, V, 1, rows, V, rows, 64, 64, None, 1.0, 0, 64, 64, 64, 64,
                                                       64, None)
    assert call(16385, 1 << 20) == -5
    assert L.dg_status_str(-5).startswith(b"input larger than the fixed scratch")
    assert call(0, 1 << 20) == -1
