#!/usr/bin/env python3
"""Denoise-step throughput on one MI355X: canvas positions denoised per second.

One step = one pass of the whole hot path over one 256-token canvas
(16 query / 8 KV heads, head_dim 256, 2048-token paged bf16 prefix,
V = 262144, d = 4096, MLP 4096 -> 1024 -> 4096):
    dg_canvas_attention -> dg_denoise_sample_sc -> dg_entropy_accept -> dg_converged -> dg_selfcond_embed_sc
(the sampling pass also writes the self-conditioning probability operand, so the logits are read
once per step)
Every input is synthetic and already resident in HBM when timing starts; the
logits of successive steps rotate through a pool of distinct sets (768 MiB,
three times the 256 MB Infinity Cache) so that no step reads them from cache.
The logits stand in for the LM head output of a real backbone.

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
           tau=0.3, max_steps=64, temperature=1.0, pool=6, seed=0, window=0, e4m3=False)
E4M3_SCALE = 2.0 ** -7      # the E4M3 table stores E / scale; E ~ N(0, 1) / 8 stays far inside +-448
KV_SCALES = (2.0 ** -4, 2.0 ** -4)   # the E4M3 cache stores K / scale, V / scale (K, V ~ N(0, 1))
PE_KERNEL = "gemm_f16_splitk_kernel<0>"
PE_KERNEL_E4M3 = "gemm_f16_e4m3_splitk_kernel"
PE_SOURCES = ("denoise_step_amd/csrc/gemm_f16.hpp",)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "pe_gemm_single_canvas_counters.json")


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


def source_sha() -> str:
    h = hashlib.sha256()
    for p in PE_SOURCES:
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
        self.q = synth.normal_torch(s, "bench.q", (C, Hq, D), 1.0, bf, dev)
        self.k = synth.normal_torch(s, "bench.k", (C, Hkv, D), 1.0, bf, dev)
        self.v = synth.normal_torch(s, "bench.v", (C, Hkv, D), 1.0, bf, dev)
        n_pages = L // ps + 2
        if c["e4m3"]:
            self.k_cache = synth.e4m3_table_torch(s, "bench.kc8", (n_pages, Hkv, ps, D), 1.0, KV_SCALES[0], dev)
            self.v_cache = synth.e4m3_table_torch(s, "bench.vc8", (n_pages, Hkv, ps, D), 1.0, KV_SCALES[1], dev)
        else:
            self.k_cache = synth.normal_torch(s, "bench.kc", (n_pages, Hkv, ps, D), 1.0, bf, dev)
            self.v_cache = synth.normal_torch(s, "bench.vc", (n_pages, Hkv, ps, D), 1.0, bf, dev)
        self.page_table = torch.as_tensor(synth.page_table(s, "bench.pages", n_pages)[: L // ps].copy(), device=dev)
        self.splits = torch.tensor([[0, L, 0, C, 0, c["window"]]], dtype=torch.int32, device=dev)
        # keys the canvas rows see together: the whole request, or the band of a sliding window
        self.key_span = L + C if c["window"] <= 0 else min(L + C, C + 2 * c["window"])
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

    def step(self, t: int, ev=None, pe_ev=None):
        """One denoise step.  ev: optional list of 6 events recorded between the calls."""
        c, dg, s = self.c, self.dg, self.state
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        if c["e4m3"]:
            dg.dg_canvas_attention_e4m3(self.q, self.k, self.v, self.k_cache, self.v_cache, *KV_SCALES,
                                        self.page_table, self.splits, c["C"], self.key_span, self.scale,
                                        out=self.att_out)
        else:
            dg.dg_canvas_attention(self.q, self.k, self.v, self.k_cache, self.v_cache, self.page_table, self.splits,
                                   c["C"], self.key_span, self.scale, out=self.att_out)
        rec(1)
        logits = self.pool[t % len(self.pool)]
        dg.dg_denoise_sample_sc(logits, c["V"], c["C"], self.seed, s["step_global"], c["temperature"], out=self.so,
                                ws=self.ws_s, sc_operand=self.sc_operand)
        rec(2)
        dg.dg_entropy_accept(self.so["entropy"], self.so["sample"], s["canvas"], c["V"], c["budget"], self.seed,
                             s["step_global"], accept=self.accept, n_accept=self.n_accept)
        rec(3)
        dg.dg_converged(self.so["argmax"], self.so["entropy"], c["V"], c["k"], c["tau"], c["max_steps"], self.seed, s)
        rec(4)
        if c["e4m3"]:
            dg.dg_selfcond_embed_sc_e4m3(self.sc_operand, c["V"], self.so["row_max"], self.so["row_lnz"], s["sc_on"],
                                         s["canvas"], self.E, E4M3_SCALE, self.prepared, c["hidden"], x_out=self.x,
                                         ws=self.ws_sc, pe_events=pe_ev)
        else:
            dg.dg_selfcond_embed_sc(self.sc_operand, c["V"], self.so["row_max"], self.so["row_lnz"], s["sc_on"],
                                    s["canvas"], self.E, self.prepared, c["hidden"], x_out=self.x, ws=self.ws_sc,
                                    pe_events=pe_ev)
        rec(5)


def call_rooflines(brk: dict, pe_ms: float, c=CFG) -> dict:
    """Per-call GPU time (events around each call in the timed region) against its own bound.

    attention: MFMA work 4 D Hq per visible (query row, key) pair: every one of the C canvas rows sees
    the L cached keys and all C canvas keys (in a sliding-window layer of window W, canvas row j at
    position L + j sees positions L + j - W .. L + j + W inside the request); sampler: the logit
    bytes (2 V per row, read once); P.E: 2 C V d FLOP on fp16 MFMA and its algorithmic bytes
    (E + P, 16-bit)."""
    C, V, d, L, W = c["B"] * c["C"], c["V"], c["d"], c["L"], c["window"]
    pairs = C * (L + C)
    if W > 0:
        pairs = c["B"] * sum(min(L + c["C"], L + j + W + 1) - max(0, L + j - W) for j in range(c["C"]))
    att_flop = 4.0 * c["D"] * c["Hq"] * pairs
    samp_bytes = 2.0 * C * V
    pe_flop = 2.0 * C * V * d
    out = {
        "canvas_attention": {"us": brk["canvas_attention"], "bound": "mfma",
                             "tflops": att_flop / (brk["canvas_attention"] * 1e-6) / 1e12},
        "denoise_sample": {"us": brk["denoise_sample"], "bound": "hbm",
                           "gbs": samp_bytes / (brk["denoise_sample"] * 1e-6) / 1e9},
        "pe_contraction": {"us": pe_ms * 1000.0, "bound": "hbm",
                           "gbs": pe_algorithmic_bytes(c) / (pe_ms * 1e-3) / 1e9,
                           "tflops": pe_flop / (pe_ms * 1e-3) / 1e12},
        "entropy_accept": {"us": brk["entropy_accept"], "bound": "latency"},
        "converged": {"us": brk["converged"], "bound": "latency"},
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
    q = f64(w.q)
    k_new, v_new = f64(w.k), f64(w.v)
    if c["e4m3"]:
        from oracle import fp8
        kc, vc = (fp8.decode_table(t.cpu().numpy(), sc) for t, sc in zip((w.k_cache, w.v_cache), KV_SCALES))
        E = fp8.decode_table(w.E.cpu().numpy(), E4M3_SCALE)
    else:
        kc, vc = f64(w.k_cache), f64(w.v_cache)
        E = w.E.float().cpu().numpy()
    pt = w.page_table.cpu().numpy()
    pool = [f64(w.pool[t % len(w.pool)]) for t in range(steps)]
    wg, wu, wd = f64(w.wg), f64(w.wu), f64(w.wd)
    threads = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else 1
    log("cpu baseline: timing the oracle")
    t0 = time.perf_counter()
    for t in range(steps):
        logits = pool[t]
        K, Vv = attention.gather_request_kv(kc, vc, k_new, v_new, pt, 0, c["L"], 0, C, 0, c["page_size"])
        group = c["Hq"] // c["Hkv"]
        mask = attention.visibility_mask(c["L"], 0, C, c["window"])
        for h in range(c["Hq"]):
            attention.dense_mask_attention(q[:, h], K[:, h // group], Vv[:, h // group], mask, 1.0 / math.sqrt(D))
        so = sampler.denoise_sample(logits, 1.0, [0], [1 + t], C)
        st = converged.LoopState(canvas=np.zeros((1, C), np.int64), prev_argmax=np.zeros((1, C), np.int64),
                                 unchanged=np.zeros(1, np.int64), step_in_block=np.ones(1, np.int64),
                                 step_global=np.ones(1, np.int64), sc_on=np.ones(1, np.uint8))
        accept.entropy_accept(so.entropy[None, :], so.sample[None, :], st.canvas, c["budget"], [0], [1 + t], V)
        converged.converged(so.argmax[None, :], so.entropy[None, :], st, c["k"], c["tau"], c["max_steps"], [0], V)
        P = selfcond.probs_from_stats(logits, 1.0, so.row_max, so.row_lnz)
        selfcond.selfcond_embed(P, st.canvas, st.sc_on, E, wg, wu, wd, C, to_bf16=True)
    dt = time.perf_counter() - t0
    cores = min(len(os.sched_getaffinity(0)), max(threads, 1))
    return dict(value=steps * C / dt, unit="positions/s", cores=cores, kind="oracle",
                sample=(f"{steps} whole steps of the {C}-position canvas ({steps * C} positions) on the host in fp64 "
                        f"numpy: attention for {C} rows x {c['Hq']} heads over {c['L'] + C} keys, the sampler over "
                        f"{C} rows of V={V} (Philox Gumbel), accept + converged, P.E + MLP against the full "
                        f"{V} x {c['d']} table; {dt:.1f} s"))


def serving_bench(policies=("deficit", "arrival")) -> dict:
    """The batched serving loop (32 requests in bursts of 8, prompts U[512, 8192], 256-token
    canvases, two blocks each, V = 262144, 8192 tokens per iteration) run to completion once per
    admission policy: deficit admission, and admitting every waiting prefill at once.  A decode
    iteration's time is what every running request waits for its next step (the decode stall).  Per iteration: one mixed
    attention launch, then sampler / accept / convergence for the denoising requests; GPU time from
    events around each iteration's launches (the host reads the commit flags once per iteration)."""
    import numpy as np
    import torch

    import synth
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
    out = {}
    for pol in policies:
        t = dict(base, k_cache=torch.zeros((sched["n_pages"], cfg["Hkv"], cfg["page_size"], cfg["D"]), dtype=bf,
                                           device=dev))
        t["v_cache"] = torch.zeros_like(t["k_cache"])
        loop = ServingLoop(cfg, sched, t, device=dev, policy=pol)
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
                       "heads_kv": cfg["Hkv"], "head_dim": cfg["D"]},
            "policies": out}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the GPU's clocks settle within the first ~50 steps (~35 ms of this load): 5 warmup steps time the
    # ramp (measured 679-687 us per step), 50 or more the steady state (648-655 us per step)
    ap.add_argument("--warmup", type=int, default=100)
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
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (no sharding, no collectives); "
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
    if args.serving:
        print(json.dumps(serving_bench()), flush=True)
        return
    w = Workload(dict(CFG, window=args.window, e4m3=args.e4m3))
    c = w.c
    log(f"warmup {args.warmup} steps")
    for t in range(args.warmup):
        w.step(t)
    torch.cuda.synchronize()
    K = args.steps
    hev = HipEvents()
    pe_ev = [(hev.create(), hev.create()) for _ in range(K)]
    # events between the calls of every timed step (on the launch stream): per-call GPU time
    call_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for t in range(K):
        w.step(args.warmup + t, ev=call_ev[t], pe_ev=pe_ev[t])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / K
    pe_ms = sum(hev.elapsed_ms(a, b) for a, b in pe_ev) / K
    names = ["canvas_attention", "denoise_sample", "entropy_accept", "converged", "selfcond_embed"]
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
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_steps)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
