#!/usr/bin/env python3
"""Denoise-step throughput on one MI355X: canvas positions denoised per second.

One step = one pass of the whole hot path over one 256-token canvas
(16 query / 8 KV heads, head_dim 256, 2048-token paged bf16 prefix,
V = 262144, d = 4096, MLP 4096 -> 1024 -> 4096):
    dg_canvas_attention -> dg_denoise_sample_sc -> dg_accept_converged -> dg_selfcond_embed_sc
(the sampling pass also writes the self-conditioning probability operand, so the logits are read
once per step)
Every input is synthetic and already resident in HBM when timing starts; the
logits of successive steps rotate through a pool of distinct sets (768 MiB,
three times the 256 MB Infinity Cache) so that no step reads them from cache.
The logits stand in for the LM head output of a real backbone.

--workload single_canvas_lmhead runs the same step from the backbone's last hidden states h
(256 x 4096 bf16): dg_lmhead_denoise_sample computes the LM head logits = h E^T on MFMA and
samples them in the same kernel (the logits never reach HBM), and dg_selfcond_embed_lm runs P.E
from its operand; its roofline is the fused LM-head kernel's (2 C V d FLOP per launch, bf16 MFMA).

Before its W warmup steps every workload first runs its own step until the GPU has been busy with
it for SETTLE_MS (~30 single-canvas steps after the host-side set-up run ~13 % slower while the
GPU's clocks come up); the JSON line records those steps as `settle_steps`.  The timed region is
exactly K steps either way.

Prints ONE JSON line (see --help).  The P.E contraction kernel, the step's
dominant launch, is timed with HIP events recorded around it on the launch
stream over the whole timed region; its roofline fraction uses the algorithmic
bytes E (V x d, 16-bit) + P (C x V, 16-bit) per launch.  The CPU oracle is
timed on a bounded sample of the same step (`cpu_baseline`).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "canvas positions denoised/sec (C=256, V=262144) + % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 / fp16
CFG = dict(B=1, C=256, L=2048, page_size=16, Hq=16, Hkv=8, D=256, V=262144, d=4096, hidden=1024, budget=8.0, k=3,
           tau=0.3, max_steps=64, temperature=1.0, pool=6, seed=0, window=0, e4m3=False, lmhead=False)
# the LM-head variant: hidden states h = a E[t] + b n (a ~ U[0, 0.4], b = 1/8) and logits = h E^T
LMHEAD = dict(scale=1.0, a_max=0.4, b=0.125)
LM_KERNEL = "lmhead_sample_kernel"
E4M3_SCALE = 2.0 ** -7      # the E4M3 table stores E / scale; E ~ N(0, 1) / 8 stays far inside +-448
KV_SCALES = (2.0 ** -4, 2.0 ** -4)   # the E4M3 cache stores K / scale, V / scale (K, V ~ N(0, 1))
PE_KERNEL = "gemm_f16_splitk_kernel<0>"
PE_KERNEL_E4M3 = "gemm_f16_e4m3_splitk_kernel"
PE_SOURCES = ("denoise_step_amd/csrc/gemm_f16.hpp",)
LM_SOURCES = ("denoise_step_amd/csrc/gemm_f16.hpp", "denoise_step_amd/csrc/lmhead.hip")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "pe_gemm_single_canvas_counters.json")
LM_COUNTERS_FILE = os.path.join(ROOT, "profiles", "lmhead_single_canvas_counters.json")
METRIC_LMHEAD = ("canvas positions denoised/sec with the LM head in the step (C=256, V=262144, d=4096) "
                 "+ % MFMA roofline")


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded (same soname, same instance)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = self.ct.c_void_p()
        assert self.hip.hipEventCreate(self.ct.byref(ev)) == 0
        return ev.value

    def elapsed_ms(self, a, b) -> float:
        ms = self.ct.c_float()
        assert self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) == 0
        return ms.value


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


SETTLE_MS = 150.0  # GPU time the workload's step runs before the warmup steps


def settle(run_one) -> int:
    """Runs the workload's step (run_one(i), i = 0, 1, ...) until SETTLE_MS of wall time has passed
    with the GPU busy on it; returns the number of steps run."""
    import torch

    n, t0 = 0, time.perf_counter()
    while True:
        run_one(n)
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1000.0 >= SETTLE_MS:
                log(f"settled after {n} steps")
                return n


def source_sha(sources=PE_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pe_algorithmic_bytes(c=CFG) -> int:
    """E read once (V x d, 16-bit, or 8-bit for the E4M3 table) + P read once (C x V, 16-bit), per
    launch (one canvas)."""
    return (1 if c["e4m3"] else 2) * c["V"] * c["d"] + 2 * c["B"] * c["C"] * c["V"]


def traffic_from_counters(per_launch_alg: int):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they match the current kernel."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    with open(COUNTERS_FILE) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha():
        return None                      # the kernel changed since the counters were taken
    return int(rec["hbm_bytes_per_dispatch"])


def lm_traffic_from_counters():
    """HBM bytes per launch of the fused LM-head kernel from the committed counter summary, if it
    matches the current sources."""
    if not os.path.exists(LM_COUNTERS_FILE):
        return None
    with open(LM_COUNTERS_FILE) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha(LM_SOURCES):
        return None
    return int(rec["hbm_bytes_per_dispatch"])


class Workload:
    """All device buffers of the single-canvas step, allocated once."""

    def __init__(self, c=CFG):
        import numpy as np
        import torch

        import denoise_step_amd as dg
        import synth
        self.c = c
        self.dg = dg
        dev = torch.device("cuda:0")
        bf = torch.bfloat16
        C, V, d, h = c["C"], c["V"], c["d"], c["hidden"]
        Hq, Hkv, D, ps, L = c["Hq"], c["Hkv"], c["D"], c["page_size"], c["L"]
        s = c["seed"]
        log("generating inputs on the GPU")
        # the attention inputs (Q/K/V rows and the paged cache) rotate through a pool of distinct sets,
        # like the logits, so a step never finds the previous step's KV in the Infinity Cache
        n_pages = L // ps + 2
        self.att_pool = []
        for i in range(c["pool"]):
            tag = (lambda name: name) if i == 0 else (lambda name, i=i: (name, i))
            a = dict(q=synth.normal_torch(s, tag("bench.q"), (C, Hq, D), 1.0, bf, dev),
                     k=synth.normal_torch(s, tag("bench.k"), (C, Hkv, D), 1.0, bf, dev),
                     v=synth.normal_torch(s, tag("bench.v"), (C, Hkv, D), 1.0, bf, dev))
            if c["e4m3"]:
                a["kc"] = synth.e4m3_table_torch(s, tag("bench.kc8"), (n_pages, Hkv, ps, D), 1.0, KV_SCALES[0], dev)
                a["vc"] = synth.e4m3_table_torch(s, tag("bench.vc8"), (n_pages, Hkv, ps, D), 1.0, KV_SCALES[1], dev)
            else:
                a["kc"] = synth.normal_torch(s, tag("bench.kc"), (n_pages, Hkv, ps, D), 1.0, bf, dev)
                a["vc"] = synth.normal_torch(s, tag("bench.vc"), (n_pages, Hkv, ps, D), 1.0, bf, dev)
            self.att_pool.append(a)
        self.q = self.att_pool[0]["q"]
        self.page_table = torch.as_tensor(synth.page_table(s, "bench.pages", n_pages)[: L // ps].copy(), device=dev)
        self.splits = torch.tensor([[0, L, 0, C, 0, c["window"]]], dtype=torch.int32, device=dev)
        # keys the canvas rows see together: the whole request, or the band of a sliding window
        self.key_span = L + C if c["window"] <= 0 else min(L + C, C + 2 * c["window"])
        if not c["lmhead"]:
            self.pool = [synth.zipf_logits_torch(s, ("bench.logits", i), C, V, dev) for i in range(c["pool"])]
        self.wg = synth.normal_torch(s, "bench.wg", (d, h), 0.02, bf, dev)
        self.wu = synth.normal_torch(s, "bench.wu", (d, h), 0.02, bf, dev)
        self.wd = synth.normal_torch(s, "bench.wd", (h, d), 0.02, bf, dev)
        if c["e4m3"]:
            self.E = synth.e4m3_table_torch(s, "bench.E8", (V, d), 1 / 8, E4M3_SCALE, dev)
            log("preparing the E4M3 E^T and fp16 MLP operand copies")
            self.prepared = dg.dg_selfcond_prepare_e4m3(self.E, self.wg, self.wu, self.wd)
        else:
            self.E = synth.normal_torch(s, "bench.E", (V, d), 1 / 8, bf, dev)
            log("preparing the fp16 operand copies")
            self.prepared = dg.dg_selfcond_prepare(self.E, self.wg, self.wu, self.wd)
        if c["lmhead"]:
            # the step starts from the backbone's last hidden states (one set per step of the pool)
            self.hpool = [synth.lmhead_hidden_torch(s, ("bench.h", i), self.E, C, LMHEAD["a_max"], LMHEAD["b"])
                          for i in range(c["pool"])]
            log("preparing the LM-head layout of the table")
            self.lm_prepared = dg.dg_lmhead_prepare(self.E)
            self.ws_lm = torch.empty(dg.dg_lmhead_ws_bytes(C, V, d), dtype=torch.uint8, device=dev)
            self.lm_operand = torch.empty(dg.dg_lmhead_operand_bytes(C, V), dtype=torch.uint8, device=dev)
        self.seed = torch.tensor([s], dtype=torch.int64, device=dev)
        z = lambda n, dt=torch.int32: torch.zeros(n, dtype=dt, device=dev)
        self.state = dict(prev_argmax=z((1, C)), unchanged=z(1), step_in_block=torch.full((1,), -1, dtype=torch.int32,
                                                                                            device=dev),
                          step_global=z(1), canvas=z((1, C)), sc_on=z(1, torch.uint8), committed=z(1, torch.uint8),
                          out_tokens=z((1, C)), steps_used=z(1), num_sampled=z(1))
        dummy_i, dummy_f = z((1, C)), torch.zeros((1, C), dtype=torch.float32, device=dev)
        dg.dg_converged(dummy_i, dummy_f, V, c["k"], c["tau"], c["max_steps"], self.seed, self.state)  # prefill
        self.att_out = torch.empty_like(self.q)
        self.so = dict(entropy=torch.empty(C, dtype=torch.float32, device=dev), argmax=z(C), sample=z(C),
                       row_max=torch.empty(C, dtype=torch.float32, device=dev),
                       row_lnz=torch.empty(C, dtype=torch.float32, device=dev))
        self.ws_s = torch.empty(dg.dg_denoise_sample_ws_bytes(C, V), dtype=torch.uint8, device=dev)
        self.ws_sc = torch.empty(dg.dg_selfcond_ws_bytes_sc(C, V, d, h), dtype=torch.uint8, device=dev)
        self.sc_operand = torch.empty(dg.dg_selfcond_operand_bytes(C, V), dtype=torch.uint8, device=dev)
        self.accept = torch.zeros((1, C), dtype=torch.uint8, device=dev)
        self.n_accept = z(1)
        self.x = torch.empty((C, d), dtype=bf, device=dev)
        self.scale = 1.0 / math.sqrt(D)
        torch.cuda.synchronize()

    def step(self, t: int, ev=None, pe_ev=None, lm_ev=None):
        """One denoise step.  ev: optional list of 5 events recorded between the calls; pe_ev / lm_ev:
        hipEvent_t pairs recorded around the P.E and the fused LM-head kernels."""
        c, dg, s = self.c, self.dg, self.state
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        a = self.att_pool[t % len(self.att_pool)]
        if c["e4m3"]:
            dg.dg_canvas_attention_e4m3(a["q"], a["k"], a["v"], a["kc"], a["vc"], *KV_SCALES,
                                        self.page_table, self.splits, c["C"], self.key_span, self.scale,
                                        out=self.att_out)
        else:
            dg.dg_canvas_attention(a["q"], a["k"], a["v"], a["kc"], a["vc"], self.page_table, self.splits,
                                   c["C"], self.key_span, self.scale, out=self.att_out)
        rec(1)
        if c["lmhead"]:
            dg.dg_lmhead_denoise_sample(self.hpool[t % len(self.hpool)], self.lm_prepared, c["V"], LMHEAD["scale"],
                                        c["C"], self.seed, s["step_global"], c["temperature"], out=self.so,
                                        ws=self.ws_lm, operand=self.lm_operand, events=lm_ev)
        else:
            logits = self.pool[t % len(self.pool)]
            dg.dg_denoise_sample_sc(logits, c["V"], c["C"], self.seed, s["step_global"], c["temperature"],
                                    out=self.so, ws=self.ws_s, sc_operand=self.sc_operand)
        rec(2)
        dg.dg_accept_converged(self.so["entropy"], self.so["sample"], self.so["argmax"], c["V"], c["budget"], c["k"],
                               c["tau"], c["max_steps"], self.seed, s, accept=self.accept, n_accept=self.n_accept)
        rec(3)
        if c["lmhead"]:
            dg.dg_selfcond_embed_lm(self.lm_operand, c["V"], self.so["row_max"], self.so["row_lnz"], s["sc_on"],
                                    s["canvas"], self.E, self.prepared, c["hidden"], x_out=self.x, ws=self.ws_sc,
                                    pe_events=pe_ev)
        elif c["e4m3"]:
            dg.dg_selfcond_embed_sc_e4m3(self.sc_operand, c["V"], self.so["row_max"], self.so["row_lnz"], s["sc_on"],
                                         s["canvas"], self.E, E4M3_SCALE, self.prepared, c["hidden"], x_out=self.x,
                                         ws=self.ws_sc, pe_events=pe_ev)
        else:
            dg.dg_selfcond_embed_sc(self.sc_operand, c["V"], self.so["row_max"], self.so["row_lnz"], s["sc_on"],
                                    s["canvas"], self.E, self.prepared, c["hidden"], x_out=self.x, ws=self.ws_sc,
                                    pe_events=pe_ev)
        rec(4)


def call_rooflines(brk: dict, pe_ms: float, c=CFG) -> dict:
    """Per-call GPU time (events around each call in the timed region) against its own bound.

    attention: MFMA work 4 D Hq per visible (query row, key) pair: every one of the C canvas rows sees
    the L cached keys and all C canvas keys (in a sliding-window layer of window W, canvas row j at
    position L + j sees positions L + j - W .. L + j + W inside the request); sampler (the fused call:
    streaming kernel + chunk merge): the logits read once (2 V per row) plus the fp16 probability
    operand it writes (2 V per row, rows padded to 256); P.E: 2 C V d FLOP on fp16 MFMA and its
    algorithmic bytes (E + P, 16-bit)."""
    C, V, d, L, W = c["B"] * c["C"], c["V"], c["d"], c["L"], c["window"]
    pairs = C * (L + C)
    if W > 0:
        pairs = c["B"] * sum(min(L + c["C"], L + j + W + 1) - max(0, L + j - W) for j in range(c["C"]))
    att_flop = 4.0 * c["D"] * c["Hq"] * pairs
    samp_bytes = 2.0 * C * V + 2.0 * (-(-C // 256) * 256) * V      # logits read once + the fp16 operand written
    pe_flop = 2.0 * C * V * d
    out = {
        "canvas_attention": {"us": brk["canvas_attention"], "bound": "mfma",
                             "tflops": att_flop / (brk["canvas_attention"] * 1e-6) / 1e12},
        "denoise_sample": {"us": brk["denoise_sample"], "bound": "hbm", "bytes": samp_bytes,
                           "gbs": samp_bytes / (brk["denoise_sample"] * 1e-6) / 1e9},
        "pe_contraction": {"us": pe_ms * 1000.0, "bound": "hbm",
                           "gbs": pe_algorithmic_bytes(c) / (pe_ms * 1e-3) / 1e9,
                           "tflops": pe_flop / (pe_ms * 1e-3) / 1e12},
        "accept_converged": {"us": brk["accept_converged"], "bound": "latency"},
    }
    for k in out.values():
        if "tflops" in k:
            k["mfma_frac"] = k["tflops"] / MFMA_PEAK_TFLOPS
        if "gbs" in k:
            k["hbm_frac"] = k["gbs"] / HBM_PEAK_GBS
    return out


def cpu_baseline(w: Workload, steps: int):
    """Time the oracle, as it stands, on `steps` whole steps of the same canvas (host cores)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import accept, attention, converged, sampler, selfcond
    c = w.c
    C, V, D = c["C"], c["V"], c["D"]
    log(f"cpu baseline: copying the inputs of {steps} steps to the host")
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    if c["e4m3"]:
        from oracle import fp8
    att = []  # each step's attention inputs (the pool set the GPU step uses)
    for t in range(steps):
        a = w.att_pool[t % len(w.att_pool)]
        if c["e4m3"]:
            kc, vc = (fp8.decode_table(x.cpu().numpy(), sc) for x, sc in zip((a["kc"], a["vc"]), KV_SCALES))
        else:
            kc, vc = f64(a["kc"]), f64(a["vc"])
        att.append((f64(a["q"]), f64(a["k"]), f64(a["v"]), kc, vc))
    if c["e4m3"]:
        E = fp8.decode_table(w.E.cpu().numpy(), E4M3_SCALE)
    else:
        E = w.E.float().cpu().numpy()
    pt = w.page_table.cpu().numpy()
    if c["lmhead"]:
        from oracle import backbone
        hpool = [f64(w.hpool[t % len(w.hpool)]) for t in range(steps)]
    else:
        pool = [f64(w.pool[t % len(w.pool)]) for t in range(steps)]
    wg, wu, wd = f64(w.wg), f64(w.wu), f64(w.wd)
    threads = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else 1
    log("cpu baseline: timing the oracle")
    oracle_samples = []
    t0 = time.perf_counter()
    for t in range(steps):
        logits = backbone.lm_head(hpool[t], E, LMHEAD["scale"]) if c["lmhead"] else pool[t]
        q, k_new, v_new, kc, vc = att[t]
        K, Vv = attention.gather_request_kv(kc, vc, k_new, v_new, pt, 0, c["L"], 0, C, 0, c["page_size"])
        group = c["Hq"] // c["Hkv"]
        mask = attention.visibility_mask(c["L"], 0, C, c["window"])
        for h in range(c["Hq"]):
            attention.dense_mask_attention(q[:, h], K[:, h // group], Vv[:, h // group], mask, 1.0 / math.sqrt(D))
        so = sampler.denoise_sample(logits, 1.0, [0], [1 + t], C)
        oracle_samples.append(so)
        st = converged.LoopState(canvas=np.zeros((1, C), np.int64), prev_argmax=np.zeros((1, C), np.int64),
                                 unchanged=np.zeros(1, np.int64), step_in_block=np.ones(1, np.int64),
                                 step_global=np.ones(1, np.int64), sc_on=np.ones(1, np.uint8))
        accept.entropy_accept(so.entropy[None, :], so.sample[None, :], st.canvas, c["budget"], [0], [1 + t], V)
        converged.converged(so.argmax[None, :], so.entropy[None, :], st, c["k"], c["tau"], c["max_steps"], [0], V)
        P = selfcond.probs_from_stats(logits, 1.0, so.row_max, so.row_lnz)
        selfcond.selfcond_embed(P, st.canvas, st.sc_on, E, wg, wu, wd, C, to_bf16=True)
    dt = time.perf_counter() - t0
    cores = min(len(os.sched_getaffinity(0)), max(threads, 1))
    w.parity = sampler_parity(w, oracle_samples)
    lm = f"the LM head h E^T ({C} x {c['d']} x {V}), " if c["lmhead"] else ""
    return dict(value=steps * C / dt, unit="positions/s", cores=cores, kind="oracle",
                sample=(f"{steps} whole steps of the {C}-position canvas ({steps * C} positions) on the host in fp64 "
                        f"numpy: attention for {C} rows x {c['Hq']} heads over {c['L'] + C} keys, {lm}the sampler "
                        f"over {C} rows of V={V} (Philox Gumbel), accept + converged, P.E + MLP against the full "
                        f"{V} x {c['d']} table; {dt:.1f} s"))


TIE_GAP, TOL_ENTROPY = 1e-5, 1e-3


def sampler_parity(w: Workload, oracle_samples) -> dict:
    """The GPU sampler (the step's fused call) on the logits, seeds and steps of the oracle's timed
    sample, compared row by row: argmax and candidate bit-exact except near-ties (top-2 gap of the
    logits or of the Gumbel keys below 1e-5, or 1e-3 for the fused LM head, counted by class),
    entropy within 1e-3 nats."""
    import numpy as np
    import torch
    dg, c = w.dg, w.c
    C, V = c["C"], c["V"]
    ties = {"argmax_gap": 0, "gumbel_key_gap": 0}
    bad = {"argmax": 0, "sample": 0, "entropy": 0}
    worst_h = 0.0
    # the fused LM head keeps fp32 logits (accumulation error ~2e-5 at |x| = 25): its tie band is 1e-3
    gap = 1e-3 if c["lmhead"] else TIE_GAP
    for t, ref in enumerate(oracle_samples):
        step = torch.full((1,), 1 + t, dtype=torch.int32, device="cuda")
        if c["lmhead"]:
            out, _ = dg.dg_lmhead_denoise_sample(w.hpool[t % len(w.hpool)], w.lm_prepared, V, LMHEAD["scale"], C,
                                                 w.seed, step, c["temperature"])
        else:
            out, _ = dg.dg_denoise_sample_sc(w.pool[t % len(w.pool)], V, C, w.seed, step, c["temperature"])
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in out.items()}
        for r in range(C):
            if got["argmax"][r] != ref.argmax[r]:
                if 0 < ref.argmax_gap[r] < gap:
                    ties["argmax_gap"] += 1
                else:
                    bad["argmax"] += 1
            if got["sample"][r] != ref.sample[r]:
                if ref.key_gap[r] < gap:
                    ties["gumbel_key_gap"] += 1
                else:
                    bad["sample"] += 1
        err = np.abs(got["entropy"].astype(np.float64) - ref.entropy)
        worst_h = max(worst_h, float(err.max()))
        bad["entropy"] += int(np.sum(err > TOL_ENTROPY))
    return {"rows": C * len(oracle_samples), "near_ties": ties, "mismatches": bad, "entropy_max_abs_err": worst_h}


def serving_bench(policies=("deficit", "arrival")) -> dict:
    """The batched serving loop (32 requests in bursts of 8, prompts U[512, 8192], 256-token
    canvases, two blocks each, V = 262144, 8192 tokens per iteration) run to completion once per
    admission policy: deficit admission, and admitting every waiting prefill at once.  A decode
    iteration's time is what every running request waits for its next step (the decode stall).  Per iteration: one mixed
    attention launch, then sampler / accept / convergence and self-conditioning (P.E over the 8192
    canvas rows, d = 4096, MLP 4096 -> 1024 -> 4096) for the denoising requests; GPU time from
    events around each iteration's launches (the host reads the commit flags once per iteration)."""
    import numpy as np
    import torch

    import synth
    from denoise_step_amd import dg_selfcond_prepare as dg_prepare
    from denoise_step_amd.serving import ServingLoop
    from synth.configs import SERVING as cfg
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    sched = synth.serving_schedule_inputs(cfg)
    s, R, C, V = cfg["seed"], cfg["R"], cfg["C"], cfg["V"]
    # admitting every waiting prefill at once can pack all prompts plus every canvas into one launch
    n = int(R * C + sched["prompt"].sum())
    log("serving: generating the Q/K/V row pools and the logit pools on the GPU")
    base = dict(q=synth.normal_torch(s, "serving.q", (n, cfg["Hq"], cfg["D"]), 1.0, bf, dev),
                k=synth.normal_torch(s, "serving.k", (n, cfg["Hkv"], cfg["D"]), 1.0, bf, dev),
                v=synth.normal_torch(s, "serving.v", (n, cfg["Hkv"], cfg["D"]), 1.0, bf, dev),
                logits=torch.stack([synth.zipf_logits_torch(s, ("serving.logits", i), R * C, V, dev)
                                    for i in range(cfg["n_pool"])]))
    E = synth.normal_torch(s, "serving.E", (V, cfg["d"]), 1 / 8, bf, dev)
    wts = [synth.normal_torch(s, tag, sh, 0.02, bf, dev)
           for tag, sh in (("serving.wg", (cfg["d"], cfg["hidden"])), ("serving.wu", (cfg["d"], cfg["hidden"])),
                           ("serving.wd", (cfg["hidden"], cfg["d"])))]
    sc = dict(E=E, prepared=dg_prepare(E, *wts), hidden=cfg["hidden"])
    out = {}
    for pol in policies:
        t = dict(base, k_cache=torch.zeros((sched["n_pages"], cfg["Hkv"], cfg["page_size"], cfg["D"]), dtype=bf,
                                           device=dev))
        t["v_cache"] = torch.zeros_like(t["k_cache"])
        loop = ServingLoop(cfg, sched, t, device=dev, policy=pol, selfcond=sc)
        log(f"serving: running the loop with {pol} admission")
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        recs = loop.run()
        wall = time.perf_counter() - wall0
        ms = np.array([r["gpu_ms"] for r in recs])
        tok = np.array([r["tokens"] for r in recs])
        den_rows = np.array([r["denoise_rows"] for r in recs])
        wait = [int(np.nonzero([rid in r["admitted"] for r in recs])[0][0]) - int(sched["arrival"][rid])
                for rid in range(R)]
        dec_ms = ms[den_rows > 0]
        out[pol] = {"iterations": len(recs), "gpu_s": float(ms.sum() / 1e3), "wall_s": wall,
                    "decode_iter_ms_p50": float(np.median(dec_ms)), "decode_iter_ms_max": float(dec_ms.max()),
                    "positions_per_s": float(den_rows.sum() / (ms.sum() / 1e3)),
                    "iter_ms_p50": float(np.median(ms)), "iter_ms_max": float(ms.max()),
                    "tokens_mean": float(tok.mean()), "tokens_max": int(tok.max()),
                    "prefill_wait_iters_mean": float(np.mean(wait)), "prefill_wait_iters_max": int(max(wait))}
    return {"metric": "serving loop: canvas positions denoised/sec with deficit token-budget admission",
            "value": out["deficit"]["positions_per_s"], "unit": "positions/s", "n_gpus": 1,
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "serving", "requests": R, "C": C, "V": V, "prompt": [cfg["P_min"], cfg["P_max"]],
                       "arrival_every": cfg["arrival_every"], "token_budget": cfg["token_budget"],
                       "blocks": cfg["blocks"], "max_steps": cfg["max_steps"], "heads_q": cfg["Hq"],
                       "heads_kv": cfg["Hkv"], "head_dim": cfg["D"], "d_embed": cfg["d"], "mlp_hidden": cfg["hidden"],
                       "self_conditioning": True},
            "policies": out}



# ------------------------------------------------------------------ batched, structured-read, block-draft lines
def _json_line(metric, value, unit, K, W, ms_total, config, roofline, cpu, extra=None, dtype="bf16"):
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": K, "warmup": W,
           "ms_per_step": ms_total / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": dtype, "data": "synthetic", "config": config, "steps_per_s": 1000.0 * K / ms_total,
           "roofline": roofline, "cpu_baseline": cpu}
    out.update(extra or {})
    return out


def _cores(threads):
    return min(len(os.sched_getaffinity(0)), max(threads, 1))


def _blas_threads():
    from threadpoolctl import threadpool_info
    info = threadpool_info()
    return max(int(i.get("num_threads", 1)) for i in info) if info else 1


def bench_batched(K: int, W: int, cpu: bool) -> dict:
    """One iteration of the batched workload as a steady-state loop: 32 requests over prefixes
    U[512, 8192] in shuffled pages, each denoising a 256-token canvas at its own step (request r at
    step 2r of its 64-step block), so a block commits every other iteration and its 256-row commit
    pass shares the next launch; per iteration one mixed attention launch (16/8 heads x 256), the
    fused sampler over 8192 rows of V = 262144, accept, convergence and self-conditioning
    (P.E over 8192 rows, d = 4096, MLP 4096 -> 1024 -> 4096).  Logits rotate through 4 sets
    (17 GB).  Dominant kernel: P.E, bound by MFMA (2 x 8192 x V x d per launch)."""
    import numpy as np
    import torch

    import denoise_step_amd as dg
    import synth
    from denoise_step_amd.serving import ServingLoop
    from synth.configs import BATCHED_LOOP
    cfg = dict(BATCHED_LOOP, n_pool=4, blocks=2)
    R, C, V, d, h = cfg["R"], cfg["C"], cfg["V"], cfg["d"], cfg["hidden"]
    Hq, Hkv, D, ps = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["page_size"]
    sched = synth.serving_schedule_inputs(cfg)
    start = synth.batched_loop_start(cfg, sched)
    n = R * C
    bf = torch.bfloat16
    log("batched: generating the row pools, caches, 4 logit sets and the table on the GPU")
    g = lambda tag, shape, std=1.0: synth.normal_torch(cfg["seed"], ("bench.batched", tag), shape, std, bf, "cuda")
    t = dict(q=g("q", (n, Hq, D)), k=g("k", (n, Hkv, D)), v=g("v", (n, Hkv, D)),
             k_cache=g("kc", (sched["n_pages"], Hkv, ps, D)), v_cache=g("vc", (sched["n_pages"], Hkv, ps, D)))
    t["logits"] = torch.empty((cfg["n_pool"], n, V), dtype=bf, device="cuda")
    for i in range(cfg["n_pool"]):
        t["logits"][i] = synth.zipf_logits_torch(cfg["seed"], ("bench.batched.logits", i), n, V, "cuda")
    E = g("E", (V, d), 1 / 8)
    w = [g(tag, sh, 0.02) for tag, sh in (("wg", (d, h)), ("wu", (d, h)), ("wd", (h, d)))]
    prepared = dg.dg_selfcond_prepare(E, *w)
    loop = ServingLoop(cfg, sched, t, selfcond=dict(E=E, prepared=prepared, hidden=h), start=start)
    n_settle = settle(loop.step)
    log(f"batched: warmup {W} iterations")
    for it in range(W):
        loop.step(n_settle + it)
    torch.cuda.synchronize()
    hev = HipEvents()
    pe_ev = [(hev.create(), hev.create()) for _ in range(K)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"batched: timing {K} iterations")
    positions = 0
    t0.record()
    for i in range(K):
        rec = loop.step(n_settle + W + i, pe_events=pe_ev[i])
        positions += rec["denoise_rows"]
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    pe_ms = sum(hev.elapsed_ms(a, b) for a, b in pe_ev) / K
    pe_flop = 2.0 * n * V * d
    achieved = pe_flop / (pe_ms * 1e-3) / 1e12
    roof = {"kernel": PE_KERNEL, "bound": "mfma", "achieved": achieved, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / MFMA_PEAK_TFLOPS, "traffic": None, "algorithmic_flop_per_launch": pe_flop,
            "avg_launch_us": pe_ms * 1000.0}
    cpu_line = None
    if cpu:
        cpu_line = _cpu_batched(loop, t, E, w, cfg, sched)
    return _json_line("canvas positions denoised/sec (batched: 32 x 256 canvases, V=262144) + % MFMA roofline",
                      positions / (ms * 1e-3), "positions/s", K, W, ms,
                      {"workload": "batched", "requests": R, "C": C, "V": V, "prefix": [cfg["P_min"], cfg["P_max"]],
                       "heads_q": Hq, "heads_kv": Hkv, "head_dim": D, "d_embed": d, "mlp_hidden": h,
                       "max_steps": cfg["max_steps"], "logit_pool": cfg["n_pool"], "self_conditioning": True},
                      roof, cpu_line, {"positions_per_iteration": positions / K, "settle_steps": n_settle})


def _cpu_batched(loop, t, E, w, cfg, sched, n_req=2):
    """The oracle on n_req requests' denoise iterations (each request's attention over its own pages,
    sampler, accept, convergence, P.E + MLP of its 256 rows) of the same loop state and inputs."""
    import numpy as np
    import torch

    from oracle import accept, attention, converged, sampler, selfcond
    C, V, D, ps = cfg["C"], cfg["V"], cfg["D"], cfg["page_size"]
    f = lambda x: x.float().cpu().numpy().astype(np.float64)
    sp, _ = loop._splits()
    host = []
    for r in range(n_req):
        i = [k for k in range(sp.shape[0]) if sp[k, 4] == sched["page0"][r]][0]
        row0, cached, nc, nv = (int(x) for x in sp[i][:4])
        p0, p1 = int(sched["page0"][r]), int(sched["page0"][r + 1])
        pt = torch.as_tensor(sched["page_table"][p0:p1].astype(np.int64), device="cuda")
        sl = slice(row0, row0 + nc + nv)
        host.append(dict(q=f(t["q"][sl]), k=f(t["k"][sl]), v=f(t["v"][sl]), kc=f(t["k_cache"][pt]),
                         vc=f(t["v_cache"][pt]), logits=f(t["logits"][0][r * C:(r + 1) * C]),
                         seed=int(sched["seeds"][r]), shape=(cached, nc, nv)))
    Eh = E.float().cpu().numpy()
    wh = [f(x) for x in w]
    log(f"cpu baseline: timing the oracle on {n_req} requests' iterations")
    threads = _blas_threads()
    t0 = time.perf_counter()
    for h in host:
        cached, nc, nv = h["shape"]
        attention.canvas_attention(h["q"], h["k"], h["v"], h["kc"], h["vc"], np.arange(h["kc"].shape[0], dtype=np.int32),
                                   [(0, cached, nc, nv, 0)], ps, 1.0 / math.sqrt(D))
        so = sampler.denoise_sample(h["logits"], 1.0, [h["seed"]], [1], C)
        st = converged.LoopState(canvas=np.zeros((1, C), np.int64), prev_argmax=np.zeros((1, C), np.int64),
                                 unchanged=np.zeros(1, np.int64), step_in_block=np.ones(1, np.int64),
                                 step_global=np.ones(1, np.int64), sc_on=np.ones(1, np.uint8))
        accept.entropy_accept(so.entropy[None, :], so.sample[None, :], st.canvas, cfg["budget"], [h["seed"]], [1], V)
        converged.converged(so.argmax[None, :], so.entropy[None, :], st, cfg["k"], cfg["tau"], cfg["max_steps"],
                            [h["seed"]], V)
        P = selfcond.probs_from_stats(h["logits"], 1.0, so.row_max, so.row_lnz)
        selfcond.selfcond_embed(P, st.canvas, st.sc_on, Eh, *wh, C, to_bf16=True)
    dt = time.perf_counter() - t0
    keys = ", ".join(f"{nc + nv} rows over {cached + nc + nv} keys" for cached, nc, nv in (h["shape"] for h in host))
    return dict(value=n_req * C / dt, unit="positions/s", cores=_cores(threads), kind="oracle",
                sample=(f"{n_req} requests' iterations of the batched loop on the host in fp64 numpy: attention "
                        f"({keys}, {cfg['Hq']} heads), the sampler over {C} rows of V={V}, accept + converged, "
                        f"P.E + MLP for {C} rows against the full table, per request; {dt:.1f} s"))


def bench_structured_read(K: int, W: int, cpu: bool) -> dict:
    """One single-pass structured read over 64 requests: each launch holds the request's final
    2048-token prompt chunk (causal rows, K/V appended to its pages) and its 256-row canvas
    (bidirectional, read-only), 16/8 heads x 256; then the allowed-choice readout of 8 slots per
    request (2-5 allowed ids) over V = 262144 slot logits.  Dominant kernel: the attention, bound by
    MFMA: 4 D Hq FLOP per visible (row, key) pair (causal triangle plus the canvas block)."""
    import numpy as np
    import torch

    import denoise_step_amd as dg
    import synth
    from synth.configs import STRUCTURED_READ as cfg
    B, C, V, nc = cfg["B"], cfg["C"], cfg["V"], cfg["n_causal"]
    Hq, Hkv, D, ps = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["page_size"]
    lay = synth.paged_layout(cfg["seed"], synth.structured_read_splits(cfg), ps, tag="bench.sread")
    bf = torch.bfloat16
    log("structured read: generating inputs on the GPU")
    g = lambda tag, shape: synth.normal_torch(cfg["seed"], ("bench.sread", tag), shape, 1.0, bf, "cuda")
    q, k, v = g("q", (lay.rows, Hq, D)), g("k", (lay.rows, Hkv, D)), g("v", (lay.rows, Hkv, D))
    kc, vc = g("kc", (lay.n_pages, Hkv, ps, D)), g("vc", (lay.n_pages, Hkv, ps, D))
    pt = torch.as_tensor(lay.page_table, device="cuda")
    sp = torch.as_tensor(lay.split_array(), device="cuda")
    rng = synth.rng_for(cfg["seed"], "bench.sread.slots")
    n_slots = B * cfg["slots"]
    counts = rng.integers(cfg["min_ids"], cfg["max_ids"] + 1, n_slots)
    offsets = torch.as_tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device="cuda")
    ids = torch.as_tensor(np.concatenate([rng.choice(V, c, replace=False) for c in counts]).astype(np.int32),
                          device="cuda")
    slot_row = torch.arange(n_slots, dtype=torch.int32, device="cuda")
    slot_logits = synth.zipf_logits_torch(cfg["seed"], "bench.sread.logits", n_slots, V, "cuda")
    out = torch.empty_like(q)
    ws = torch.empty(max(1, dg.dg_canvas_attention_ws_bytes(B, lay.rows, nc + C, nc + C, Hq, Hkv, D, dg.DG_BF16)),
                     dtype=torch.uint8, device="cuda")
    qv = torch.empty(int(counts.sum()), dtype=torch.float32, device="cuda")
    ans = torch.empty(n_slots, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)

    def one(ev=None):
        if ev is not None:
            ev[0].record()
        dg.dg_canvas_attention(q, k, v, kc, vc, pt, sp, nc + C, nc + C, scale, out=out, ws=ws)
        if ev is not None:
            ev[1].record()
        dg.dg_allowed_probs(slot_logits, V, slot_row, offsets, ids, 1.0, q=qv, answer=ans)

    n_settle = settle(lambda i: one())
    log(f"structured read: warmup {W}")
    for _ in range(W):
        one()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(K):
        one(evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    att_ms = sum(a.elapsed_time(b) for a, b in evs) / K
    pairs = B * (nc * (nc + 1) // 2 + C * (nc + C))
    flop = 4.0 * D * Hq * pairs
    achieved = flop / (att_ms * 1e-3) / 1e12
    roof = {"kernel": "attend_mfma16_kernel<256, false>", "bound": "mfma", "achieved": achieved,
            "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MFMA_PEAK_TFLOPS, "traffic": None,
            "algorithmic_flop_per_launch": flop, "avg_launch_us": att_ms * 1000.0}
    cpu_line = None
    if cpu:
        from oracle import attention, readout
        f = lambda x: x.float().cpu().numpy().astype(np.float64)
        r0, nr = int(lay.row0[0]), nc + C
        pages = torch.as_tensor(lay.pages_of(0).astype(np.int64), device="cuda")
        qh, kh, vh = f(q[r0:r0 + nr]), f(k[r0:r0 + nr]), f(v[r0:r0 + nr])
        kch, vch = f(kc[pages]), f(vc[pages])
        sl = f(slot_logits[:cfg["slots"]])
        off = offsets[:cfg["slots"] + 1].cpu().numpy()
        idh = ids[:int(off[-1])].cpu().numpy()
        threads = _blas_threads()
        log("cpu baseline: timing the oracle on one request")
        tc = time.perf_counter()
        attention.canvas_attention(qh, kh, vh, kch, vch, np.arange(kch.shape[0], dtype=np.int32), [(0, 0, nc, C, 0)],
                                   ps, scale)
        readout.allowed_probs(sl, off, idh)
        dt = time.perf_counter() - tc
        cpu_line = dict(value=C / dt, unit="positions/s", cores=_cores(threads), kind="oracle",
                        sample=(f"one request of the launch on the host in fp64 numpy: attention for its {nc} causal "
                                f"+ {C} canvas rows x {Hq} heads (K/V appended), the readout of its {cfg['slots']} "
                                f"slots; {dt:.1f} s"))
    return _json_line("canvas positions read/sec (structured read: 64 x (2048 causal + 256 canvas), V=262144) "
                      "+ % MFMA roofline", B * C * K / (ms * 1e-3), "positions/s", K, W, ms,
                      {"workload": "structured_read", "requests": B, "causal_rows": nc, "C": C, "V": V,
                       "heads_q": Hq, "heads_kv": Hkv, "head_dim": D, "slots": cfg["slots"]},
                      roof, cpu_line, {"attention_us": att_ms * 1000.0, "settle_steps": n_settle})


def bench_block_draft(K: int, W: int, cpu: bool) -> dict:
    """One parallel-drafting pass: 5 draft layers of attention (128 requests x 16 draft rows over
    injected context U[256, 4096], 32 query / 8 KV heads x 128, each layer its own K/V), the
    argmax-only sampler over 2048 x 151936 bf16 logits and greedy verification of the 128 blocks
    against targets whose first mismatch is geometric(0.2).  Dominant work: the attention, bound by
    HBM (the context K/V is read once per layer)."""
    import numpy as np
    import torch

    import denoise_step_amd as dg
    import synth
    from synth.configs import BLOCK_DRAFT as cfg
    B, L16, V, layers = cfg["B"], cfg["block"], cfg["V"], cfg["layers"]
    Hq, Hkv, D, ps = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["page_size"]
    bf = torch.bfloat16
    log("block draft: generating 5 layers of context K/V and the logits on the GPU")
    lays, L = [], []
    for layer in range(layers):
        lay = synth.paged_layout(cfg["seed"], synth.block_draft_splits(cfg), ps, tag=("bench.draft", layer))
        g = lambda tag, shape: synth.normal_torch(cfg["seed"], ("bench.draft", layer, tag), shape, 1.0, bf, "cuda")
        L.append(dict(q=g("q", (lay.rows, Hq, D)), k=g("k", (lay.rows, Hkv, D)), v=g("v", (lay.rows, Hkv, D)),
                      kc=g("kc", (lay.n_pages, Hkv, ps, D)), vc=g("vc", (lay.n_pages, Hkv, ps, D)),
                      pt=torch.as_tensor(lay.page_table, device="cuda"),
                      sp=torch.as_tensor(lay.split_array(), device="cuda"),
                      max_keys=max(s.cached + s.n_causal + s.n_canvas for s in lay.splits)))
        L[-1]["out"] = torch.empty_like(L[-1]["q"])
        L[-1]["ws"] = torch.empty(max(1, dg.dg_canvas_attention_ws_bytes(B, lay.rows, L16, L[-1]["max_keys"], Hq, Hkv,
                                                                        D, dg.DG_BF16)), dtype=torch.uint8,
                                  device="cuda")
        lays.append(lay)
    logits = synth.zipf_logits_torch(cfg["seed"], "bench.draft.logits", B * L16, V, "cuda")
    amax = torch.empty(B * L16, dtype=torch.int32, device="cuda")
    ws_s = torch.empty(dg.dg_denoise_sample_ws_bytes(B * L16, V), dtype=torch.uint8, device="cuda")
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)

    def one(ev=None):
        if ev is not None:
            ev[0].record()
        for x in L:
            dg.dg_canvas_attention(x["q"], x["k"], x["v"], x["kc"], x["vc"], x["pt"], x["sp"], L16, x["max_keys"],
                                   scale, out=x["out"], ws=x["ws"])
        if ev is not None:
            ev[1].record()
        dg.dg_denoise_sample(logits, V, L16, None, None, 1.0, argmax_only=True, out=dict(argmax=amax), ws=ws_s)
        dg.dg_verify_prefix(amax.view(B, L16), target, accepted=acc)

    # targets: the draft argmax with its first mismatch at a geometric(0.2) offset (later ids random)
    dg.dg_denoise_sample(logits, V, L16, None, None, 1.0, argmax_only=True, out=dict(argmax=amax), ws=ws_s)
    draft = amax.view(B, L16).cpu().numpy()
    rng = synth.rng_for(cfg["seed"], "bench.draft.targets")
    gmm = rng.geometric(cfg["p_mismatch"], B) - 1
    tgt = draft.copy()
    for b in range(B):
        if gmm[b] < L16:
            tgt[b, gmm[b]] = (draft[b, gmm[b]] + 1 + rng.integers(0, V - 1)) % V
            tgt[b, gmm[b] + 1:] = rng.integers(0, V, L16 - 1 - gmm[b])
    target = torch.as_tensor(tgt, device="cuda")
    n_settle = settle(lambda i: one())
    log(f"block draft: warmup {W}")
    for _ in range(W):
        one()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(K):
        one(evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    att_ms = sum(a.elapsed_time(b) for a, b in evs) / K
    kv_bytes = sum(2 * 2 * Hkv * D * sum(s.cached + s.n_causal + s.n_canvas for s in lay.splits) for lay in lays)
    achieved = kv_bytes / (att_ms * 1e-3) / 1e9
    roof = {"kernel": "attend_mfma16_kernel<128, false> (5 layers)", "bound": "hbm", "achieved": achieved,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
            "algorithmic_bytes_per_pass": kv_bytes, "avg_pass_attention_us": att_ms * 1000.0}
    assert np.array_equal(acc.cpu().numpy(), np.minimum(gmm, L16)), "verification disagrees with its construction"
    cpu_line = None
    if cpu:
        from oracle import attention, verify
        f = lambda x: x.float().cpu().numpy().astype(np.float64)
        reqs = tuple(range(16))
        host = []
        for x, lay in zip(L, lays):
            for r in reqs:
                s_ = lay.splits[r]
                r0, nr = int(lay.row0[r]), s_.n_causal + s_.n_canvas
                pages = torch.as_tensor(lay.pages_of(r).astype(np.int64), device="cuda")
                host.append((f(x["q"][r0:r0 + nr]), f(x["k"][r0:r0 + nr]), f(x["v"][r0:r0 + nr]), f(x["kc"][pages]),
                             f(x["vc"][pages]), s_))
        hl = f(logits[:len(reqs) * L16])
        threads = _blas_threads()
        log(f"cpu baseline: timing the oracle on {len(reqs)} requests")
        tc = time.perf_counter()
        for qh, kh, vh, kch, vch, s_ in host:
            attention.canvas_attention(qh, kh, vh, kch, vch, np.arange(kch.shape[0], dtype=np.int32),
                                       [(0, s_.cached, s_.n_causal, s_.n_canvas, 0)], ps, scale)
        am = np.argmax(hl, axis=1).reshape(len(reqs), L16)
        verify.verify_prefix(am, tgt[:len(reqs)])
        dt = time.perf_counter() - tc
        cpu_line = dict(value=len(reqs) * L16 / dt, unit="draft positions/s", cores=_cores(threads), kind="oracle",
                        sample=(f"{len(reqs)} of the 128 requests on the host in fp64 numpy: 5 layers of attention "
                                f"for their 16 draft rows x {Hq} heads over their injected context, the argmax of "
                                f"their {len(reqs) * L16} logit rows of V={V}, verification; {dt:.1f} s"))
    return _json_line("draft positions/sec (block draft: 128 x 16 positions, 5 layers, V=151936) + % HBM roofline",
                      B * L16 * K / (ms * 1e-3), "draft positions/s", K, W, ms,
                      {"workload": "block_draft", "requests": B, "block": L16, "layers": layers,
                       "context": [cfg["L_min"], cfg["L_max"]], "heads_q": Hq, "heads_kv": Hkv, "head_dim": D,
                       "V": V}, roof, cpu_line,
                      {"attention_us_per_pass": att_ms * 1000.0,
                       "accepted_mean": float(np.minimum(gmm, L16).mean()), "settle_steps": n_settle})

def pe_probe(passes: int = 3) -> dict:
    """Self-conditioning passes of the batched configuration (32 x 256 rows, V 262144, d 4096) on
    synthetic inputs: N(0, 2^2) logits through dg_denoise_sample_sc for the operand, then
    dg_selfcond_embed_sc `passes` times.  Few kernels run besides the M = 8192 P.E GEMM, so profiler
    counters (which serialise every kernel) take seconds, where the batched loop's would not."""
    import torch
    import denoise_step_amd as dg
    import synth
    from synth.configs import BATCHED as c
    B, C, V, d, hid, s = c["B"], c["C"], c["V"], c["d"], c["hidden"], c["seed"]
    bf, dev = torch.bfloat16, "cuda"
    log("pe probe: inputs")
    logits = synth.normal_torch(s, "pe_probe.logits", (B * C, V), 2.0, bf, dev)
    E = synth.normal_torch(s, "pe_probe.E", (V, d), 0.02, bf, dev)
    wg = synth.normal_torch(s, "pe_probe.wg", (d, hid), 0.02, bf, dev)
    wu = synth.normal_torch(s, "pe_probe.wu", (d, hid), 0.02, bf, dev)
    wd = synth.normal_torch(s, "pe_probe.wd", (hid, d), 0.02, bf, dev)
    seed = torch.arange(B, dtype=torch.int64, device=dev) * 7 + 1
    step = torch.zeros(B, dtype=torch.int32, device=dev)
    sc_on = torch.ones(B, dtype=torch.uint8, device=dev)
    canvas = torch.as_tensor(synth.rng_for(s, "pe_probe.canvas").integers(0, V, (B, C)).astype("int32"), device=dev)
    prepared = dg.dg_selfcond_prepare(E, wg, wu, wd)
    out, op = dg.dg_denoise_sample_sc(logits, V, C, seed, step)
    torch.cuda.synchronize()
    del logits
    x, ms = None, []
    for i in range(passes):
        t0 = time.perf_counter()
        x = dg.dg_selfcond_embed_sc(op, V, out["row_max"], out["row_lnz"], sc_on, canvas, E, prepared, hid, x_out=x)
        torch.cuda.synchronize()
        ms.append((time.perf_counter() - t0) * 1e3)
        log(f"pe probe: pass {i} {ms[-1]:.2f} ms")
    return {"pe_probe_rows": B * C, "V": V, "d": d, "passes": passes, "ms_per_pass": [round(m, 3) for m in ms]}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=("single_canvas", "single_canvas_lmhead", "batched", "structured_read",
                                           "block_draft"),
                    default="single_canvas",
                    help="single_canvas: one 256-token canvas step (default); single_canvas_lmhead: the same step "
                         "from the backbone's hidden states, the LM head fused with the sampler; batched: one "
                         "iteration of the 32-request batched loop; structured_read: one 64-request single-pass "
                         "read launch; block_draft: one 5-layer parallel draft + argmax + verify pass")
    ap.add_argument("--cpu-steps", type=int, default=2, help="whole steps of the canvas in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--serving", action="store_true",
                    help="run the batched serving loop with deficit admission (and admit-on-arrival for "
                         "comparison) instead of the single-canvas step; prints its own JSON line")
    ap.add_argument("--e4m3", action="store_true",
                    help="run the step with an E4M3 (FP8) paged KV cache and embedding table instead of bf16 ones")
    ap.add_argument("--window", type=int, default=0,
                    help="run the step as a sliding-window layer of this window (0: full attention)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run three plain 1 GiB device copies (reference for HBM counter calibration)")
    ap.add_argument("--pe-probe", action="store_true",
                    help="only run three batched self-conditioning passes (P.E over 32 x 256 rows, the MLP) on "
                         "synthetic inputs: a short run for the counters of the M = 8192 P.E GEMM")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (no sharding, no collectives); "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        x = torch.empty(2 ** 30, dtype=torch.uint8, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 2 ** 30, "copy_probe_bytes_written": 2 ** 30, "calls": 3}))
        return
    import denoise_step_amd as dg
    dg.lib()
    if args.pe_probe:
        print(json.dumps(pe_probe()), flush=True)
        return
    if args.serving:
        print(json.dumps(serving_bench()), flush=True)
        return
    if args.workload not in ("single_canvas", "single_canvas_lmhead"):
        fn = {"batched": bench_batched, "structured_read": bench_structured_read,
              "block_draft": bench_block_draft}[args.workload]
        print(json.dumps(fn(args.steps, args.warmup, not args.no_cpu_baseline)), flush=True)
        return
    lmhead = args.workload == "single_canvas_lmhead"
    if lmhead and (args.e4m3 or args.window):
        print("the LM-head step runs with the bf16 table and full attention", file=sys.stderr)
        sys.exit(2)
    w = Workload(dict(CFG, window=args.window, e4m3=args.e4m3, lmhead=lmhead))
    c = w.c
    n_settle = settle(w.step)
    log(f"warmup {args.warmup} steps")
    for t in range(args.warmup):
        w.step(t)
    torch.cuda.synchronize()
    K = args.steps
    hev = HipEvents()
    pe_ev = [(hev.create(), hev.create()) for _ in range(K)]
    lm_ev = [(hev.create(), hev.create()) for _ in range(K)] if lmhead else [None] * K
    # events between the calls of every timed step (on the launch stream): per-call GPU time
    call_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for t in range(K):
        w.step(args.warmup + t, ev=call_ev[t], pe_ev=pe_ev[t], lm_ev=lm_ev[t])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / K
    pe_ms = sum(hev.elapsed_ms(a, b) for a, b in pe_ev) / K
    names = ["canvas_attention", "denoise_sample", "accept_converged", "selfcond_embed"]
    brk = {n: sum(ev[i].elapsed_time(ev[i + 1]) for ev in call_ev) * 1000.0 / K for i, n in enumerate(names)}
    alg = pe_algorithmic_bytes(c)
    achieved = alg / (pe_ms * 1e-3) / 1e9
    positions = c["B"] * c["C"]
    kernels = call_rooflines(brk, pe_ms, c)
    result = {
        "metric": METRIC,
        "value": positions * K / (ms_total * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_steps": n_settle,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if not c["e4m3"] else "bf16 (E4M3 KV cache and table; bf16 / fp16 MFMA)",
        "data": "synthetic",
        "config": {"workload": "single_canvas" + (f"_window{c['window']}" if c["window"] > 0 else "")
                   + ("_e4m3" if c["e4m3"] else ""), "B": c["B"], "C": c["C"], "V": c["V"], "prefix": c["L"],
                   "heads_q": c["Hq"], "heads_kv": c["Hkv"], "head_dim": c["D"], "page_size": c["page_size"],
                   "d_embed": c["d"], "mlp_hidden": c["hidden"], "logit_pool": c["pool"], "window": c["window"]},
        "steps_per_s": 1000.0 / ms_step,
        "wall_s_timed_region": wall,
        "roofline": {"kernel": PE_KERNEL_E4M3 if c["e4m3"] else PE_KERNEL, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None if c["e4m3"] else traffic_from_counters(alg),
                     "algorithmic_bytes_per_launch": alg, "avg_launch_us": pe_ms * 1000.0,
                     "source_sha": source_sha()},
        "breakdown_us": brk,
        "kernels": kernels,
    }
    if c["e4m3"]:
        # with the E4M3 table P.E moves half the bytes for the same fp16 MFMA work (455 FLOP/B, above
        # the 315 FLOP/B ridge): its bound is the MFMA peak
        pe_flop = 2.0 * c["B"] * c["C"] * c["V"] * c["d"]
        tf = pe_flop / (pe_ms * 1e-3) / 1e12
        result["roofline"] = {"kernel": PE_KERNEL_E4M3, "bound": "mfma", "achieved": tf, "peak": MFMA_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": tf / MFMA_PEAK_TFLOPS, "traffic": None,
                              "algorithmic_flop_per_launch": pe_flop, "algorithmic_bytes_per_launch": alg,
                              "avg_launch_us": pe_ms * 1000.0, "source_sha": source_sha()}
    if lmhead:
        # the dominant kernel is the fused LM head: 2 C V d FLOP on bf16 MFMA per launch
        lm_ms = sum(hev.elapsed_ms(a, b) for a, b in lm_ev) / K
        lm_flop = 2.0 * positions * c["V"] * c["d"]
        lm_tf = lm_flop / (lm_ms * 1e-3) / 1e12
        result["metric"] = METRIC_LMHEAD
        result["config"]["workload"] = "single_canvas_lmhead"
        result["config"]["lm_head"] = {"scale": LMHEAD["scale"], "hidden": "a E[t] + b n, a ~ U[0, 0.4], b = 1/8"}
        del result["config"]["logit_pool"]
        result["roofline"] = {"kernel": LM_KERNEL, "bound": "mfma", "achieved": lm_tf, "peak": MFMA_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": lm_tf / MFMA_PEAK_TFLOPS,
                              "traffic": lm_traffic_from_counters(),
                              "algorithmic_flop_per_launch": lm_flop, "avg_launch_us": lm_ms * 1000.0,
                              "source_sha": source_sha(LM_SOURCES)}
        result["breakdown_us"]["lmhead_denoise_sample"] = result["breakdown_us"].pop("denoise_sample")
        kernels["lmhead_sample_kernel"] = {"us": lm_ms * 1000.0, "bound": "mfma", "tflops": lm_tf,
                                           "mfma_frac": lm_tf / MFMA_PEAK_TFLOPS}
        del kernels["denoise_sample"]
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_steps)
        result["parity"] = w.parity
        result["near_ties"] = w.parity["near_ties"]
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
