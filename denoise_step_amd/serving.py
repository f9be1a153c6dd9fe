"""A batched serving loop around the denoise step, with deficit token-budget admission.

Each iteration (Sangam page, section on the deficit token-budget scheduler, for the admission;
DiffusionGemma/vLLM page, sections "Two modes, one set of weights" and "Dynamic per-sequence
causal attention", for the phases that share one launch; section "Self-conditioning" for the
feedback into the next step):
  * decode work is scheduled first: every request that denoises a canvas (C canvas rows) or runs
    the commit pass of its last block (C causal rows);
  * dg_deficit_admit decides whether the prefill at the head of the arrival queue enters, whole;
  * one dg_canvas_attention launch covers every scheduled request in its own phase (prefill and
    commit rows causal with K/V appended to the request's pages, canvas rows bidirectional);
  * the denoising requests run dg_denoise_sample -> dg_accept_converged (acceptance + convergence in
    one launch); a request admitted this iteration gets its first random canvas from its prefill case;
  * with self-conditioning, the sampling pass also writes the probability operand
    (dg_denoise_sample_sc) and dg_selfcond_embed_sc turns it into the next step's canvas
    embedding x_next = E[canvas] + (sc_on ? MLP(softmax . E) : 0), after dg_converged has set the
    new canvas and sc_on (off for a block that just committed and restarted);
  * a committed block is followed by its commit pass in the next iteration; after `blocks` blocks
    the request leaves.
A steady-state start (`start`) puts every request in the denoising phase from the first iteration,
over a prefix already in its pages and at its own step (the batched workload: requests at different
steps, each block committing at its cap, running its commit pass and restarting).
Activations and logits come from synthetic pools (no trained backbone): the loop exercises the
scheduling, the launch composition, the paged cache and the per-request state.  All arithmetic
runs in libdg; this module keeps the request phases and sequences the calls.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import (dg_accept_converged, dg_canvas_attention, dg_converged, dg_deficit_admit, dg_denoise_sample,
               dg_denoise_sample_sc, dg_denoise_sample_ws_bytes, dg_selfcond_embed_sc, dg_selfcond_operand_bytes,
               dg_selfcond_ws_bytes_sc)

WAITING, PREFILL, DENOISE, COMMIT, DONE = range(5)


class ServingLoop:
    def __init__(self, cfg: dict, sched: dict, tensors: dict, device="cuda", policy: str = "deficit",
                 selfcond: dict | None = None, start: dict | None = None):
        """tensors: q/k/v row pools, k_cache/v_cache, logits pools [n_pool, R*C, V] (torch on `device`).
        selfcond: dict(E [V, d] bf16, prepared = dg_selfcond_prepare(E, ...), hidden): run the
        self-conditioning of every denoise iteration (x_next in self.x).
        start: dict(cached, step_in_block, step_global), one int per request: every request starts
        denoising over `cached` tokens already in its pages, with a canvas drawn by dg_converged's
        prefill case at step_global - 1 and then those counters (sc_on = step_in_block > 0)."""
        self.cfg, self.sched, self.policy = cfg, sched, policy
        dev = torch.device(device)
        self.dev = dev
        self.t = tensors
        R, C = cfg["R"], cfg["C"]
        z = lambda shape, dt=torch.int32: torch.zeros(shape, dtype=dt, device=dev)
        self.state = dict(prev_argmax=z((R, C)), unchanged=z(R),
                          step_in_block=torch.full((R,), -1, dtype=torch.int32, device=dev), step_global=z(R),
                          canvas=z((R, C)), sc_on=z(R, torch.uint8), committed=z(R, torch.uint8),
                          out_tokens=z((R, C)), steps_used=z(R), num_sampled=z(R))
        self.seed = torch.as_tensor(sched["seeds"].astype(np.int64), device=dev)
        self.page_table = torch.as_tensor(sched["page_table"], dtype=torch.int32, device=dev)
        self.accept = z((R, C), torch.uint8)
        self.n_accept = z(R)
        self.phase = np.full(R, WAITING)
        self.cached = np.zeros(R, np.int64)
        self.blocks_done = np.zeros(R, np.int64)
        self.queue = []
        self.deficit = 0
        self.scale = 1.0 / math.sqrt(cfg["D"])
        V = cfg["V"]
        self.so = dict(entropy=torch.empty(R * C, dtype=torch.float32, device=dev), argmax=z(R * C),
                       sample=z(R * C), row_max=torch.empty(R * C, dtype=torch.float32, device=dev),
                       row_lnz=torch.empty(R * C, dtype=torch.float32, device=dev))
        self.ws_s = torch.empty(dg_denoise_sample_ws_bytes(R * C, V), dtype=torch.uint8, device=dev)
        self.sc = selfcond
        if selfcond is not None:
            E = selfcond["E"]
            # zero-filled once: rows of requests that do not denoise keep finite (earlier) values
            self.operand = torch.zeros(dg_selfcond_operand_bytes(R * C, V), dtype=torch.uint8, device=dev)
            self.ws_sc = torch.empty(dg_selfcond_ws_bytes_sc(R * C, V, E.shape[1], selfcond["hidden"]),
                                     dtype=torch.uint8, device=dev)
            self.x = torch.zeros((R * C, E.shape[1]), dtype=E.dtype, device=dev)
        if start is not None:
            st = self.state
            st["step_global"].copy_(torch.as_tensor(np.asarray(start["step_global"]) - 1, dtype=torch.int32))
            zi = torch.zeros((R, C), dtype=torch.int32, device=dev)
            dg_converged(zi, torch.zeros((R, C), dtype=torch.float32, device=dev), V, cfg["k"], cfg["tau"],
                         cfg["max_steps"], self.seed, st)                  # prefill case: first canvases
            sib = np.asarray(start["step_in_block"], np.int32)
            st["step_in_block"].copy_(torch.as_tensor(sib))
            st["sc_on"].copy_(torch.as_tensor((sib > 0).astype(np.uint8)))
            self.phase[:] = DENOISE
            self.cached[:] = np.asarray(start["cached"], np.int64)
        self.steady = start is not None
        self.last = {}

    def _schedule(self, it: int):
        """Phases of this iteration: arrivals join the queue, decode work first, then admission."""
        cfg, s = self.cfg, self.sched
        if not self.steady:                       # a steady-state start has admitted every request
            for r in np.nonzero(s["arrival"] == it)[0]:
                self.queue.append(int(r))
        decode = int(np.sum((self.phase == DENOISE) | (self.phase == COMMIT))) * cfg["C"]
        sizes = [int(s["prompt"][r]) for r in self.queue]
        if self.policy == "deficit":
            n, self.deficit, tokens = dg_deficit_admit(cfg["token_budget"], decode, sizes, self.deficit)
        else:                      # admit every waiting prefill at once (no budget)
            n, tokens = len(sizes), decode + sum(sizes)
        admitted = self.queue[:n]
        self.queue = self.queue[n:]
        for r in admitted:
            self.phase[r] = PREFILL
        return admitted, tokens

    def _splits(self):
        """dg_split rows (request order) for every request scheduled this iteration."""
        C, rows, out = self.cfg["C"], 0, []
        for r in range(self.cfg["R"]):
            ph = self.phase[r]
            if ph == PREFILL:
                nc, nv, cached = int(self.sched["prompt"][r]), 0, 0
            elif ph == DENOISE:
                nc, nv, cached = 0, C, int(self.cached[r])
            elif ph == COMMIT:
                nc, nv, cached = C, 0, int(self.cached[r])
            else:
                continue
            out.append([rows, cached, nc, nv, int(self.sched["page0"][r]), 0])
            rows += nc + nv
        return np.array(out, np.int32).reshape(-1, 6), rows

    def step(self, it: int, record: bool = False, pe_events=None):
        """One iteration.  pe_events: optional (start, stop) hipEvent_t handles recorded around the
        P.E kernel of the self-conditioning call (it then runs only in iterations with denoising)."""
        cfg = self.cfg
        R, C, V = cfg["R"], cfg["C"], cfg["V"]
        admitted, tokens = self._schedule(it)
        sp, rows = self._splits()
        if rows > self.t["q"].shape[0]:
            raise ValueError(f"iteration {it} packs {rows} rows but the Q/K/V pools hold {self.t['q'].shape[0]}")
        rec = dict(iteration=it, admitted=admitted, tokens=tokens, deficit=self.deficit, rows=rows,
                   denoise_rows=int(np.sum(self.phase == DENOISE)) * C)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        if rows > 0:
            spl = torch.as_tensor(sp, device=self.dev)
            max_rows = int(np.max(sp[:, 2] + sp[:, 3]))
            max_keys = int(np.max(sp[:, 1] + sp[:, 2] + sp[:, 3]))
            att = dg_canvas_attention(self.t["q"][:rows], self.t["k"][:rows], self.t["v"][:rows], self.t["k_cache"],
                                      self.t["v_cache"], self.page_table, spl, max_rows, max_keys, self.scale)
            if record:
                rec["splits"] = sp.copy()
                rec["attention"] = att.float().cpu().numpy()
        den = torch.as_tensor((self.phase == DENOISE).astype(np.uint8), device=self.dev)
        pre = torch.as_tensor(((self.phase == DENOISE) | (self.phase == PREFILL)).astype(np.uint8), device=self.dev)
        st = self.state
        denoising = bool((self.phase == DENOISE).any())
        if denoising:
            logits = self.t["logits"][it % cfg["n_pool"]]
            step_now = st["step_global"].clone()
            so = self.so
            if self.sc is not None:
                dg_denoise_sample_sc(logits, V, C, self.seed, step_now, cfg["temperature"], active=den, out=so,
                                     ws=self.ws_s, sc_operand=self.operand)
            else:
                dg_denoise_sample(logits, V, C, self.seed, step_now, cfg["temperature"], active=den, out=so,
                                  ws=self.ws_s)
            argmax, entropy, sample = so["argmax"].view(R, C), so["entropy"].view(R, C), so["sample"].view(R, C)
        else:
            argmax = sample = torch.zeros((R, C), dtype=torch.int32, device=self.dev)
            entropy = torch.zeros((R, C), dtype=torch.float32, device=self.dev)
        if bool(((self.phase == DENOISE) | (self.phase == PREFILL)).any()):
            st["committed"].zero_()
            # denoising requests: acceptance then the convergence test; admitted ones: the prefill case
            dg_accept_converged(entropy, sample, argmax, V, cfg["budget"], cfg["k"], cfg["tau"], cfg["max_steps"],
                                self.seed, st, active=pre, accept=self.accept, n_accept=self.n_accept)
        if denoising and self.sc is not None:
            dg_selfcond_embed_sc(self.operand, V, self.so["row_max"], self.so["row_lnz"], st["sc_on"], st["canvas"],
                                 self.sc["E"], self.sc["prepared"], self.sc["hidden"], x_out=self.x, ws=self.ws_sc,
                                 pe_events=pe_events)
        ev1.record()
        self.last = dict(denoise=self.phase == DENOISE, attention=att if rows > 0 else None)
        committed = st["committed"].cpu().numpy().astype(bool) & (self.phase == DENOISE)
        rec["gpu_ms"] = (ev0, ev1)
        rec["committed"] = {int(r): st["out_tokens"][r].cpu().numpy().copy() for r in np.nonzero(committed)[0]}
        if record:
            rec["canvas"] = st["canvas"].cpu().numpy().copy()
            if self.sc is not None and denoising:
                rec["x_next"] = self.x.float().cpu().numpy().copy()
        # phase transitions for the next iteration
        for r in range(R):
            ph = self.phase[r]
            if ph == PREFILL:
                self.cached[r] = int(self.sched["prompt"][r])
                self.phase[r] = DENOISE
            elif ph == COMMIT:
                self.cached[r] += C
                self.phase[r] = DENOISE if self.blocks_done[r] < cfg["blocks"] else DONE
            elif ph == DENOISE and committed[r]:
                self.blocks_done[r] += 1
                self.phase[r] = COMMIT
        return rec

    def checkpoint(self) -> dict:
        """The loop's state between two iterations: the host scheduling state (phases, cached tokens,
        finished blocks, queue, deficit) and copies of every device buffer a later iteration reads (the
        per-request state, the paged KV cache, the sampler outputs, and with self-conditioning the
        probability operand and the next-step embedding).  The library keeps no state of its own and
        every random draw is keyed by (seed, step, position), so restoring this into a loop over the same
        schedule and input pools continues it exactly."""
        dev = {f"state.{k}": v.clone() for k, v in self.state.items()}
        dev.update({f"so.{k}": v.clone() for k, v in self.so.items()})
        dev.update(k_cache=self.t["k_cache"].clone(), v_cache=self.t["v_cache"].clone())
        if self.sc is not None:
            dev.update(operand=self.operand.clone(), x=self.x.clone())
        host = dict(phase=self.phase.copy(), cached=self.cached.copy(), blocks_done=self.blocks_done.copy(),
                    queue=list(self.queue), deficit=self.deficit, steady=self.steady)
        return dict(host=host, device=dev)

    def restore(self, ck: dict) -> None:
        """Continue from a checkpoint() of a loop with the same configuration, schedule and input pools
        (device buffers are copied into this loop's own)."""
        dev = ck["device"]
        for k, v in self.state.items():
            v.copy_(dev[f"state.{k}"])
        for k, v in self.so.items():
            v.copy_(dev[f"so.{k}"])
        self.t["k_cache"].copy_(dev["k_cache"])
        self.t["v_cache"].copy_(dev["v_cache"])
        if self.sc is not None:
            self.operand.copy_(dev["operand"])
            self.x.copy_(dev["x"])
        h = ck["host"]
        self.phase, self.cached, self.blocks_done = h["phase"].copy(), h["cached"].copy(), h["blocks_done"].copy()
        self.queue, self.deficit, self.steady = list(h["queue"]), h["deficit"], h["steady"]

    def run(self, max_iters: int = 100000, record: bool = False, first: int = 0):
        log = []
        for it in range(first, first + max_iters):
            if np.all(self.phase == DONE):
                break
            log.append(self.step(it, record))
        torch.cuda.synchronize()
        for rec in log:
            a, b = rec.pop("gpu_ms")
            rec["gpu_ms"] = a.elapsed_time(b)
        return log
