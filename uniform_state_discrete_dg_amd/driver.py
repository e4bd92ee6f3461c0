"""Host loop over the C ABI: the pages' generation procedure.

[P2] update loop: start from a random canvas and repeat a fixed number of
whole-canvas denoising passes.  [P3] §5.3 scheduler: a step budget, a
temperature that falls as the steps count down, and an adaptive stop.
[P3] §5.2 / [P1] block diffusion: a finished canvas is appended to the KV
cache by a causal prefill and the next canvas starts fresh.

Only scalars are computed here (the temperature of each step); every tensor
operation is a libdgdenoise call.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

from . import binding as B


def temperature(kind: str, T0: float, T1: float, s: int, S: int) -> float:
    """Temperature of step s of S (host double, passed to the library as float).

    t = s / (S - 1); linear T0 + (T1 - T0) t; cosine T1 + (T0 - T1)(1 + cos(pi t)) / 2.
    """
    t = s / (S - 1) if S > 1 else 0.0
    if kind == "linear":
        return T0 + (T1 - T0) * t
    if kind == "cosine":
        return T1 + (T0 - T1) * 0.5 * (1.0 + math.cos(math.pi * t))
    return T0


@dataclass
class CanvasResult:
    tokens: torch.Tensor
    steps: int
    stop_reason: str
    stats: list = field(default_factory=list)


class Denoiser:
    """One model on one GPU: weights, a KV cache, a canvas and a workspace."""

    def __init__(self, c: dict, inp: dict, capacity: int | None = None, max_prefill: int = 0,
                 accept_rule: int = B.DG_ACCEPT_SUM_MINUS_MAX, device="cuda",
                 logits_dump: bool = False, candidate_rule: int = B.DG_CANDIDATE_ARGMAX,
                 sampler: int = B.DG_SAMPLER_UNIFORM):
        self.c = c
        self.cfg = B.make_config(c, accept_rule=accept_rule, candidate_rule=candidate_rule, sampler=sampler)
        st = B.dg_validate_config(self.cfg)
        if st != B.DG_OK:
            raise B.DgError("dg_validate_config", st)
        self.w = B.DeviceWeights(self.cfg, inp, device)
        cap = capacity if capacity is not None else c.get("cap", c["L"])
        has_prefix = c["L"] > 0 and inp["k_prefix"].shape[1] > 0
        self.cache = B.DeviceCache(self.cfg, max(cap, 1), device,
                                   inp["k_prefix"] if has_prefix else None,
                                   inp["v_prefix"] if has_prefix else None)
        self.canvas = B.DeviceCanvas(self.cfg, device)
        self.ws = B.workspace(self.cfg, max_prefill, device, logits_dump=logits_dump)

    # --- thin wrappers --------------------------------------------------------
    def init_canvas(self, seed: int, canvas_id: int) -> None:
        B.dg_canvas_init(self.cfg, self.canvas.s, seed, canvas_id)

    def step(self, T: float, gamma: float) -> None:
        B.dg_denoise_step(self.cfg, self.w.s, self.cache.s, self.canvas.s, T, gamma, self.ws)

    def should_stop(self, stable_steps: int):
        return B.dg_should_stop(self.cfg, self.canvas.s, stable_steps)

    def prefill(self, tokens: torch.Tensor, attn_out: torch.Tensor | None = None) -> None:
        B.dg_prefill_append(self.cfg, self.w.s, self.cache.s, tokens, int(tokens.numel()),
                            attn_out, self.ws)

    # --- the pages' loops -------------------------------------------------------
    def run_canvas(self, seed: int, canvas_id: int, steps: int, sched: str, T0: float, T1: float,
                   gamma: float, stop: bool, stable_n: int) -> CanvasResult:
        self.init_canvas(seed, canvas_id)
        reason = "budget"
        n = 0
        stats = []
        for s in range(steps):
            self.step(temperature(sched, T0, T1, s, steps), gamma)
            n += 1
            if stop:
                halt, st = self.should_stop(stable_n)
                stats.append(st)
                if halt:
                    reason = "confident" if st.allconf else ("unmasked" if st.masked == 0 else "stable")
                    break
        return CanvasResult(self.canvas.tokens.clone(), n, reason, stats)

    def run_canvas_native(self, seed: int, canvas_id: int, steps: int, sched: str, T0: float,
                          T1: float, gamma: float, stop: bool, stable_n: int) -> CanvasResult:
        """The same loop inside the library (dg_run_canvas): one call, one
        status readback per step when the adaptive stop is on."""
        temps = [temperature(sched, T0, T1, s, steps) for s in range(steps)]
        n, stopped = B.dg_run_canvas(self.cfg, self.w.s, self.cache.s, self.canvas.s, seed, canvas_id,
                                     temps, gamma, stop, stable_n, self.ws)
        reason = "budget"
        if stopped:
            st = self.canvas.status.cpu()
            reason = ("confident" if int(st[B.DG_ST_ALLCONF]) else
                      "unmasked" if int(st[B.DG_ST_MASKED]) == 0 else "stable")
        return CanvasResult(self.canvas.tokens.clone(), n, reason, [])

    def block_diffusion(self, prompt: torch.Tensor, canvases: int, seed: int, steps: int,
                        sched: str, T0: float, T1: float, gamma: float, stop: bool,
                        stable_n: int) -> list[CanvasResult]:
        """Prefill the prompt, then denoise `canvases` canvases, appending each
        finished one to the cache (causal incremental prefill)."""
        if prompt.numel():
            self.prefill(prompt)
        out = []
        for b in range(canvases):
            r = self.run_canvas_native(seed, b, steps, sched, T0, T1, gamma, stop, stable_n)
            self.prefill(self.canvas.tokens)
            out.append(r)
        return out
