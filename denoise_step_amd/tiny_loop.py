"""The tiny closed denoise loop on the GPU, driven through the C ABI.

One request, one fp32 layer (the two-mode backbone of the DiffusionGemma/vLLM
page, section "Two modes, one set of weights"): encoder prefill of the prompt
(causal, K/V written), prefill case of the sampler (random canvas), denoise
steps (decoder pass -> dg_denoise_sample -> dg_accept_converged (acceptance + convergence)
-> dg_selfcond_embed) until the canvas commits, then the encoder commit pass
that appends the block's K/V.  Every step of the arithmetic runs in libdg;
this module only allocates tensors and sequences the calls.
"""
from __future__ import annotations

import math

import torch

from . import (dg_accept_converged, dg_canvas_attention, dg_converged, dg_denoise_sample, dg_gather_rows, dg_linear,
               dg_selfcond_embed)


class TinyLoop:
    def __init__(self, cfg: dict, weights: dict, device="cuda"):
        self.cfg = cfg
        dev = torch.device(device)
        self.dev = dev
        f = lambda a: torch.as_tensor(a, dtype=torch.float32, device=dev).contiguous()
        self.E = f(weights["E"])
        self.w = {k: f(weights[k]) for k in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")}
        self.prefix = torch.as_tensor(weights["prefix"], dtype=torch.int32, device=dev)
        self.page_table = torch.as_tensor(weights["page_table"], dtype=torch.int32, device=dev)
        n_pages = int(weights["n_pages_total"])
        Hkv, D, ps = cfg["Hkv"], cfg["D"], cfg["page_size"]
        self.k_cache = torch.zeros((n_pages, Hkv, ps, D), dtype=torch.float32, device=dev)
        self.v_cache = torch.zeros_like(self.k_cache)
        self.scale = float(weights["logit_scale"])
        self.seed = torch.tensor([int(weights["seed64"])], dtype=torch.int64, device=dev)
        C = cfg["C"]
        z = lambda n, dt=torch.int32: torch.zeros(n, dtype=dt, device=dev)
        self.state = dict(prev_argmax=z((1, C)), unchanged=z(1), step_in_block=torch.full((1,), -1, dtype=torch.int32,
                                                                                            device=dev),
                          step_global=z(1), canvas=z((1, C)), sc_on=z(1, torch.uint8), committed=z(1, torch.uint8),
                          out_tokens=z((1, C)), steps_used=z(1), num_sampled=z(1))

    def _layer(self, x, cached, n_causal, n_canvas):
        cfg = self.cfg
        rows = x.shape[0]
        q = dg_linear(x, self.w["wq"]).view(rows, cfg["Hq"], cfg["D"])
        k = dg_linear(x, self.w["wk"]).view(rows, cfg["Hkv"], cfg["D"])
        v = dg_linear(x, self.w["wv"]).view(rows, cfg["Hkv"], cfg["D"])
        splits = torch.tensor([[0, cached, n_causal, n_canvas, 0, 0]], dtype=torch.int32, device=self.dev)
        o = dg_canvas_attention(q, k, v, self.k_cache, self.v_cache, self.page_table, splits, rows,
                                cached + n_causal + n_canvas, 1.0 / math.sqrt(cfg["D"]))
        return dg_linear(o.view(rows, cfg["Hq"] * cfg["D"]), self.w["wo"], residual=x)

    def run(self, record: bool = False) -> dict:
        cfg = self.cfg
        C, V, P0 = cfg["C"], cfg["V"], cfg["prefix"]
        s = self.state
        x = dg_gather_rows(self.E, self.prefix)
        self._layer(x, 0, P0, 0)                                   # encoder prefill: K/V written
        dummy_i = torch.zeros((1, C), dtype=torch.int32, device=self.dev)
        dummy_f = torch.zeros((1, C), dtype=torch.float32, device=self.dev)
        dg_converged(dummy_i, dummy_f, V, cfg["k"], cfg["tau"], cfg["max_steps"], self.seed, s)  # prefill case
        x = dg_gather_rows(self.E, s["canvas"].view(-1))
        traj = []
        n_acc = torch.zeros(1, dtype=torch.int32, device=self.dev)
        accept = torch.zeros((1, C), dtype=torch.uint8, device=self.dev)
        result = None
        for _t in range(cfg["max_steps"]):
            step_now = s["step_global"].clone()
            h = self._layer(x, P0, 0, C)                            # decoder pass over the canvas
            logits = dg_linear(h, self.E, trans_b=True, alpha=self.scale)
            so = dg_denoise_sample(logits, V, C, self.seed, step_now, cfg["temperature"])
            dg_accept_converged(so["entropy"], so["sample"], so["argmax"], V, cfg["budget"], cfg["k"], cfg["tau"],
                                cfg["max_steps"], self.seed, s, accept=accept, n_accept=n_acc)
            x = dg_selfcond_embed(logits, V, so["row_max"], so["row_lnz"], s["sc_on"], s["canvas"], self.E,
                                  self.w["w_gate"], self.w["w_up"], self.w["w_down"], None, cfg["temperature"])
            committed = bool(s["committed"].item())
            if record:
                traj.append(dict(entropy=so["entropy"].cpu().numpy(), argmax=so["argmax"].cpu().numpy(),
                                 sample=so["sample"].cpu().numpy(), n_accept=int(n_acc.item()),
                                 canvas=s["canvas"][0].cpu().numpy(), committed=int(committed),
                                 x_next=x.cpu().numpy(), logits=logits.cpu().numpy()))
            if committed:
                result = dict(tokens=s["out_tokens"][0].cpu().numpy(), steps_used=int(s["steps_used"].item()))
                break
        xc = dg_gather_rows(self.E, s["out_tokens"].view(-1))
        self._layer(xc, P0, C, 0)                                  # encoder commit pass: block K/V appended
        result.update(traj=traj, k_cache=self.k_cache.cpu().numpy(), v_cache=self.v_cache.cpu().numpy())
        return result
