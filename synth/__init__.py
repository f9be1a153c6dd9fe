"""Seeded synthetic inputs shared by the oracle-side tests and the GPU-side tests.

This module only *generates* inputs (numpy PCG64 streams, fixed recipes); it
holds none of the denoise step's arithmetic.  Both the CPU oracle (through the
tests) and the HIP path (through the binding) consume exactly the bytes made
here, so a parity test compares the two on identical inputs.

Storage conventions
  * bf16 tensors are returned as ``uint16`` arrays holding the bf16 bit pattern
    (the top half of an IEEE fp32, rounded to nearest even).
  * fp32 tensors are ``float32`` arrays.

Recipes (all values drawn from ``numpy.random.Generator(PCG64(seed))`` with a
per-tensor sub-seed, so changing one tensor never shifts another):
  * logits: ``sqrt(3) * z - alpha_r * 1.1 * ln(1 + rank_r(i))`` with
    ``z ~ N(0, 1)``, ``alpha_r ~ U(0, 3)`` per row and ``rank_r`` a random
    permutation of ``0..V-1`` per row: a N(0, 3) body plus a per-row Zipf(1.1)
    bias of random strength, so row entropies spread from near 0 to ~11 nats.
  * embedding table E: ``N(0, 1) / 8``.
  * MLP / projection weights: ``N(0, 0.02^2)``.
  * attention Q/K/V: ``N(0, 1)``.
  * page tables: a shuffled free list of physical pages.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "rng_for", "f32_to_bf16_bits", "bf16_bits_to_f32", "normal_bf16", "normal_f32",
    "zipf_logits_bf16", "zipf_logits_f32", "page_table", "SplitSpec", "attention_problem",
    "PagedAttentionProblem",
]


def rng_for(seed: int, *tags) -> np.random.Generator:
    """Independent PCG64 stream for (seed, tags...)."""
    h = hashlib.sha256(repr((int(seed),) + tuple(tags)).encode()).digest()
    return np.random.Generator(np.random.PCG64(int.from_bytes(h[:16], "little")))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(seed: int, tag: str, shape, std: float = 1.0) -> np.ndarray:
    rng = rng_for(seed, tag)
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):
        n = min(step, flat.size - s)
        flat[s:s + n] = rng.standard_normal(n, dtype=np.float32) * np.float32(std)
    return out


def normal_bf16(seed: int, tag: str, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) rounded to bf16; generated in chunks so large tables stay cheap."""
    rng = rng_for(seed, tag)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):
        n = min(step, flat.size - s)
        flat[s:s + n] = f32_to_bf16_bits(rng.standard_normal(n, dtype=np.float32) * np.float32(std))
    return out


def _zipf_rows(seed: int, tag: str, rows: int, V: int, alpha_max: float) -> np.ndarray:
    rng = rng_for(seed, tag)
    alpha = rng.uniform(0.0, alpha_max, size=rows)
    base = (-1.1 * np.log1p(np.arange(V, dtype=np.float64))).astype(np.float32)
    out = np.empty((rows, V), dtype=np.float32)
    for r in range(rows):
        z = rng.standard_normal(V, dtype=np.float32)
        perm = rng.permutation(V)
        out[r] = np.float32(np.sqrt(3.0)) * z + np.float32(alpha[r]) * base[perm]
    return out


def zipf_logits_f32(seed: int, tag: str, rows: int, V: int, alpha_max: float = 3.0) -> np.ndarray:
    return _zipf_rows(seed, tag, rows, V, alpha_max)


def zipf_logits_bf16(seed: int, tag: str, rows: int, V: int, alpha_max: float = 3.0) -> np.ndarray:
    """bf16 logit rows (uint16 bits), N(0, 3) body + per-row Zipf(1.1) bias of strength U(0, alpha_max)."""
    out = np.empty((rows, V), dtype=np.uint16)
    chunk = max(1, (1 << 23) // max(V, 1))
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        out[r0:r1] = f32_to_bf16_bits(_zipf_rows(seed, (tag, r0), r1 - r0, V, alpha_max))
    return out


def page_table(seed: int, tag: str, n_pages_total: int) -> np.ndarray:
    """A shuffled free list of physical page ids (int32)."""
    return rng_for(seed, tag).permutation(n_pages_total).astype(np.int32)


@dataclass
class SplitSpec:
    """One request's row split for one attention launch.

    cached   : tokens already resident in the request's pages
    n_causal : causal rows (prompt chunk / commit pass) in this launch
    n_canvas : bidirectional canvas rows in this launch
    """
    cached: int
    n_causal: int
    n_canvas: int


@dataclass
class PagedAttentionProblem:
    Hq: int
    Hkv: int
    D: int
    page_size: int
    splits: list            # list[SplitSpec]
    row0: np.ndarray        # int32 [n_req]
    page0: np.ndarray       # int32 [n_req]
    page_table: np.ndarray  # int32 [sum pages]
    q: np.ndarray           # [rows, Hq, D]   (uint16 bf16 bits or float32)
    k: np.ndarray           # [rows, Hkv, D]
    v: np.ndarray           # [rows, Hkv, D]
    k_cache: np.ndarray     # [n_pages, Hkv, page_size, D]
    v_cache: np.ndarray
    dtype: str = "bf16"
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return int(self.q.shape[0])


@dataclass
class PagedLayout:
    """Row and page placement of one attention launch (no tensor data)."""
    splits: list            # list[SplitSpec]
    row0: np.ndarray        # int32 [n_req]
    page0: np.ndarray       # int32 [n_req]
    page_table: np.ndarray  # int32 [sum of the requests' pages]
    n_pages: int            # physical pages in the pool (owned + spare)
    rows: int               # packed rows of the launch
    page_size: int

    def split_array(self) -> np.ndarray:
        """[n_req, 6] int32 rows of (row0, cached, n_causal, n_canvas, page0, window = 0)."""
        return np.array([[self.row0[i], s.cached, s.n_causal, s.n_canvas, self.page0[i], 0]
                         for i, s in enumerate(self.splits)], np.int32).reshape(-1, 6)

    def pages_of(self, i: int) -> np.ndarray:
        """Physical page ids of request i, in position order."""
        s = self.splits[i]
        n = max(1, -(-(s.cached + s.n_causal) // self.page_size))
        return self.page_table[self.page0[i]:self.page0[i] + n]


def paged_layout(seed: int, splits, page_size: int = 16, spare_pages: int = 3, tag: str = "attn") -> PagedLayout:
    """Each request owns ceil((cached + n_causal) / page_size) pages (room for the causal rows'
    K/V to be appended), drawn from one global shuffled pool with ``spare_pages`` extra pages that
    no request owns; rows are packed request after request."""
    splits = [s if isinstance(s, SplitSpec) else SplitSpec(*s) for s in splits]
    need = [max(1, -(-(s.cached + s.n_causal) // page_size)) for s in splits]
    n_pages = int(sum(need)) + spare_pages
    pool = page_table(seed, (tag, "pool"), n_pages)
    page0 = np.zeros(len(splits), np.int32)
    row0 = np.zeros(len(splits), np.int32)
    tbl = []
    r = 0
    p = 0
    for i, (s, n) in enumerate(zip(splits, need)):
        page0[i] = p
        row0[i] = r
        tbl.extend(pool[p:p + n].tolist())
        p += n
        r += s.n_causal + s.n_canvas
    return PagedLayout(splits=splits, row0=row0, page0=page0, page_table=np.asarray(tbl, np.int32),
                       n_pages=n_pages, rows=r, page_size=page_size)


def attention_problem(seed: int, splits, Hq: int, Hkv: int, D: int, page_size: int = 16,
                      dtype: str = "bf16", spare_pages: int = 3, tag: str = "attn") -> PagedAttentionProblem:
    """Random Q/K/V, a paged cache filled for each request's cached prefix, and shuffled page tables
    (layout of paged_layout; the spare pages stay as random junk so reading a wrong page shows up)."""
    lay = paged_layout(seed, splits, page_size, spare_pages, tag)
    rows, n_pages = lay.rows, lay.n_pages
    gen = normal_bf16 if dtype == "bf16" else normal_f32
    q = gen(seed, (tag, "q"), (rows, Hq, D))
    k = gen(seed, (tag, "k"), (rows, Hkv, D))
    v = gen(seed, (tag, "v"), (rows, Hkv, D))
    kc = gen(seed, (tag, "kc"), (n_pages, Hkv, page_size, D))
    vc = gen(seed, (tag, "vc"), (n_pages, Hkv, page_size, D))
    return PagedAttentionProblem(Hq=Hq, Hkv=Hkv, D=D, page_size=page_size, splits=lay.splits,
                                 row0=lay.row0, page0=lay.page0, page_table=lay.page_table,
                                 q=q, k=k, v=v, k_cache=kc, v_cache=vc, dtype=dtype)


def batched_splits(cfg: dict, commit_requests=(5, 21)) -> list:
    """Batched serving snapshot: prefixes U{L_min..L_max}; the listed requests are in the launch
    right after their commit (256 causal rows appended, no canvas rows), the others denoise a
    canvas of C rows."""
    L = rng_for(cfg["seed"], "batched.L").integers(cfg["L_min"], cfg["L_max"] + 1, cfg["B"])
    return [SplitSpec(int(L[r]), cfg["C"], 0) if r in commit_requests else SplitSpec(int(L[r]), 0, cfg["C"])
            for r in range(cfg["B"])]


def structured_read_splits(cfg: dict) -> list:
    """Final prompt chunk (causal rows, nothing cached before it) plus the canvas, per request."""
    return [SplitSpec(0, cfg["n_causal"], cfg["C"]) for _ in range(cfg["B"])]


def block_draft_splits(cfg: dict) -> list:
    """Injected context U{L_min..L_max} per request plus the draft block as canvas rows."""
    L = rng_for(cfg["seed"], "block_draft.L").integers(cfg["L_min"], cfg["L_max"] + 1, cfg["B"])
    return [SplitSpec(int(L[r]), 0, cfg["block"]) for r in range(cfg["B"])]


def tiny_loop_inputs(cfg: dict, variant_scale: float | None = None) -> dict:
    """Weights, embedding table, prefix tokens and page table of the one-layer fp32 tiny loop.

    ``variant_scale`` only relabels the logit scale (test-only variants that exercise
    acceptance and convergence); the arrays are the same for every variant.
    """
    s, d, V = cfg["seed"], cfg["d"], cfg["V"]
    HqD, HkvD, h = cfg["Hq"] * cfg["D"], cfg["Hkv"] * cfg["D"], cfg["hidden"]
    n_tok = cfg["prefix"] + cfg["C"]
    n_pages = -(-n_tok // cfg["page_size"])
    return dict(
        E=normal_f32(s, "tiny.E", (V, d), cfg["e_std"]),
        wq=normal_f32(s, "tiny.wq", (d, HqD), cfg["w_std"]),
        wk=normal_f32(s, "tiny.wk", (d, HkvD), cfg["w_std"]),
        wv=normal_f32(s, "tiny.wv", (d, HkvD), cfg["w_std"]),
        wo=normal_f32(s, "tiny.wo", (HqD, d), cfg["w_std"]),
        w_gate=normal_f32(s, "tiny.wg", (d, h), cfg["w_std"]),
        w_up=normal_f32(s, "tiny.wu", (d, h), cfg["w_std"]),
        w_down=normal_f32(s, "tiny.wd", (h, d), cfg["w_std"]),
        prefix=rng_for(s, "tiny.prefix").integers(0, V, cfg["prefix"]).astype(np.int32),
        page_table=page_table(s, "tiny.pages", n_pages + 2)[:n_pages].copy(),
        n_pages_total=n_pages + 2,
        logit_scale=float(cfg["logit_scale"] if variant_scale is None else variant_scale),
        seed64=np.uint64(s),
    )


# ---------------------------------------------------------------- large inputs generated on the GPU
# Full-size tables (a 262144 x 4096 embedding table, thousands of 262144-wide logit rows) are
# drawn with torch's seeded device generator instead of numpy, then copied to the host where
# the oracle needs them.  Same recipes as above; values are deterministic for a given seed,
# shape and device type.

def _torch_gen(seed: int, tag, device):
    import torch
    h = hashlib.sha256(repr((int(seed), "torch") + (tag if isinstance(tag, tuple) else (tag,))).encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return g


def normal_torch(seed: int, tag, shape, std: float, dtype, device, chunk_rows: int = 1 << 14):
    """N(0, std^2) of `shape`, rounded to `dtype` (torch.bfloat16 or float32), generated on `device`."""
    import torch
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    g = _torch_gen(seed, tag, device)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = (torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device) * std).to(dtype)
    return out


def zipf_logits_torch(seed: int, tag, rows: int, V: int, device, alpha_max: float = 3.0, dtype=None,
                      chunk_rows: int = 64):
    """Same recipe as zipf_logits_bf16: sqrt(3) z - alpha_r * 1.1 * ln(1 + rank_r(i)), bf16."""
    import torch
    dtype = dtype or torch.bfloat16
    g = _torch_gen(seed, tag, device)
    alpha = torch.rand(rows, generator=g, device=device) * alpha_max
    base = -1.1 * torch.log1p(torch.arange(V, device=device, dtype=torch.float32))
    out = torch.empty((rows, V), dtype=dtype, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        z = torch.randn((r1 - r0, V), generator=g, device=device)
        perm = torch.argsort(torch.rand((r1 - r0, V), generator=g, device=device), dim=1)
        out[r0:r1] = (np.sqrt(3.0) * z + alpha[r0:r1, None] * base[perm]).to(dtype)
    return out


def serving_schedule_inputs(cfg: dict) -> dict:
    """Prompt lengths, arrival iterations and the paged layout of the serving loop.

    Request r arrives at iteration (r // burst) * arrival_every (bursts of `burst` requests, 1 if
    unset) with a prompt of U[P_min, P_max] tokens and
    owns ceil((P + blocks * C) / page_size) pages (prompt plus every committed block), a contiguous
    slice of one shuffled page table with two spare pages that nobody owns."""
    s, R, ps = cfg["seed"], cfg["R"], cfg["page_size"]
    P = rng_for(s, "serving.prompts").integers(cfg["P_min"], cfg["P_max"] + 1, R).astype(np.int64)
    need = [-(-(int(p) + cfg["blocks"] * cfg["C"]) // ps) for p in P]
    n_pages = int(sum(need)) + 2
    tbl = page_table(s, "serving.pages", n_pages)
    page0 = np.concatenate([[0], np.cumsum(need)[:-1]]).astype(np.int32)
    arrival = (np.arange(R, dtype=np.int64) // cfg.get("burst", 1)) * cfg["arrival_every"]
    return dict(prompt=P, arrival=arrival, page0=page0,
                page_table=tbl[:int(sum(need))].copy(), n_pages=n_pages,
                seeds=np.array([(s << 20) + r for r in range(R)], np.uint64),
                max_rows=int(R * cfg["C"] + cfg["P_max"]))


def serving_small_tensors(cfg: dict, sched: dict) -> dict:
    """Host arrays (bf16 bits) for the small serving loop: Q/K/V row pools, initial caches, logit pools."""
    s, R, C, V = cfg["seed"], cfg["R"], cfg["C"], cfg["V"]
    n = sched["max_rows"]
    Hq, Hkv, D, ps = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["page_size"]
    return dict(
        q=normal_bf16(s, "serving.q", (n, Hq, D)),
        k=normal_bf16(s, "serving.k", (n, Hkv, D)),
        v=normal_bf16(s, "serving.v", (n, Hkv, D)),
        k_cache=normal_bf16(s, "serving.kc", (sched["n_pages"], Hkv, ps, D)),
        v_cache=normal_bf16(s, "serving.vc", (sched["n_pages"], Hkv, ps, D)),
        logits=np.stack([zipf_logits_bf16(s, ("serving.logits", i), R * C, V) for i in range(cfg["n_pool"])]),
    )


def e4m3_table(seed: int, tag, shape, std: float, scale: float) -> np.ndarray:
    """OCP E4M3 codes (uint8) of N(0, std^2) / scale values, rounded to nearest by torch's
    float8_e4m3fn conversion: a table whose values are scale * decode(codes)."""
    import torch
    x = normal_f32(seed, tag, shape, std) / np.float32(scale)
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_table_torch(seed: int, tag, shape, std: float, scale: float, device, chunk_rows: int = 1 << 14):
    """e4m3_table drawn with torch's device generator (full-size tables), as a uint8 tensor."""
    import torch
    out = torch.empty(shape, dtype=torch.uint8, device=device)
    flat = out.view(shape[0], -1)
    g = _torch_gen(seed, tag, device)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device) * (std / scale)
        flat[r0:r1] = x.to(torch.float8_e4m3fn).view(torch.uint8)
    return out


def batched_loop_start(cfg: dict, sched: dict) -> dict:
    """Steady-state start of the batched loop: request r holds its prompt as a cached prefix and sits
    at step 2r of its block (mod the step cap) and global step 2r + 1 (its first canvas drawn at
    global step 2r)."""
    R = cfg["R"]
    r = np.arange(R, dtype=np.int64)
    return dict(cached=sched["prompt"].copy(), step_in_block=(2 * r) % cfg["max_steps"], step_global=2 * r + 1)


# ---------------------------------------------------------------- LM-head inputs
# A hidden state with a planted direction: h_r = a_r E[t_r] + b n_r with a_r ~ U[0, a_max],
# t_r uniform over the vocabulary and n_r ~ N(0, I), rounded to bf16.  With E ~ N(0, 1/64) the
# logit of t_r stands about a_r d / 64 above the others, whose spread is about
# sqrt(a_r^2 d / 4096 + b^2 d / 64): rows range from diffuse (a_r ~ 0) to peaked.

def lmhead_hidden_bf16(seed: int, tag, E_bits: np.ndarray, rows: int, a_max: float, b: float) -> np.ndarray:
    """h [rows][d] as bf16 bits from the bf16 table E_bits [V][d] (numpy)."""
    g = rng_for(seed, tag, "h")
    V, d = E_bits.shape
    a = g.random(rows) * a_max
    t = g.integers(0, V, rows)
    h = a[:, None] * bf16_bits_to_f32(E_bits[t]).astype(np.float64) + b * g.standard_normal((rows, d))
    return f32_to_bf16_bits(h.astype(np.float32))


def lmhead_hidden_torch(seed: int, tag, E, rows: int, a_max: float, b: float):
    """The same recipe drawn with torch's device generator from a device bf16 table E [V][d]."""
    import torch
    g = _torch_gen(seed, (tag, "h") if not isinstance(tag, tuple) else tag + ("h",), E.device)
    V, d = E.shape
    a = torch.rand(rows, generator=g, device=E.device) * a_max
    t = torch.randint(0, V, (rows,), generator=g, device=E.device)
    n = torch.randn((rows, d), generator=g, device=E.device)
    return (a[:, None] * E[t].float() + b * n).to(torch.bfloat16)

