"""A MoE layer driven through the C ABI: buffers come from torch (device memory
only), every computation is a call into ``libmoe_mi355x.so``.

Forward:  moe_route_permute (plain routing; else moe_route -> moe_permute)
          -> moe_expert_ffn -> moe_combine
          (+ aux_balance_loss when a balance or z-loss coefficient is set);
          expert choice: moe_route_expert_choice -> moe_expert_ffn -> moe_combine
Backward: moe_backward (with the aux-loss logit gradient as d_logits_extra)
"""
from __future__ import annotations

import os
from dataclasses import dataclass

import torch

from . import _lib as L


@dataclass
class LayerSpec:
    T: int
    D: int
    E: int
    K: int
    F: int
    lo: int = 0
    hi: int = -1
    n_shared: int = 0
    score: int = L.MOE_SCORE_SOFTMAX
    gating: int = L.MOE_GATE_RENORM
    dtype: int = L.MOE_BF16
    cap: float = 0.0
    alpha: float = 0.0
    zlam: float = 0.0
    seq_len: int = 0          # sequence-wise balance loss over sequences of this length (0: off)
    seq_alpha: float = 0.0
    bias_gamma: float = 0.0   # load-driven selection-bias step after each routing (0: off)
    routing: int = L.MOE_TOKEN_CHOICE  # MOE_EXPERT_CHOICE: experts pick tokens (gating A)

    def config(self) -> L.MoeConfig:
        return L.make_config(self.T, self.D, self.E, self.K, self.F, self.lo,
                             self.E if self.hi < 0 else self.hi, self.n_shared, self.score,
                             self.gating, self.dtype, self.cap, self.routing)

    @property
    def expert_choice(self) -> bool:
        return self.routing == L.MOE_EXPERT_CHOICE

    @property
    def width(self) -> int:
        """Slots per token in the slot tables: K, or E under expert choice."""
        return self.E if self.expert_choice else self.K

    @property
    def groups(self) -> int:
        return (self.E if self.hi < 0 else self.hi) - self.lo + self.n_shared

    @staticmethod
    def from_workload(wl, **over) -> "LayerSpec":
        kw = dict(T=wl.T, D=wl.D, E=wl.E, K=wl.K, F=wl.F, lo=wl.lo, hi=wl.hi,
                  n_shared=wl.n_shared, score=wl.score, gating=wl.gating, dtype=wl.dtype,
                  cap=wl.cap, alpha=wl.alpha, zlam=wl.zlam)
        kw.update(over)
        return LayerSpec(**kw)


class MoELayer:
    def __init__(self, spec: LayerSpec, w_r, w_gate, w_up, w_down, r_bias=None, sel_bias=None,
                 device="cuda", w_noise=None):
        self.spec = spec
        self.cfg = spec.config()
        self.dev = torch.device(device)
        s = spec
        tdt = torch.bfloat16 if s.dtype == L.MOE_BF16 else torch.float32
        self.tdt = tdt
        self.w_r, self.w_gate, self.w_up, self.w_down = w_r, w_gate, w_up, w_down
        self.r_bias, self.sel_bias = r_bias, sel_bias
        self.w_noise = w_noise  # noisy top-K: [E][D] fp32 noise router, or None
        self.jitter = None      # router-logit jitter of the last forward ([T][E] fp32)
        rows = max(L.rows_max(self.cfg), 1)
        T1 = max(s.T, 1)
        G = s.groups
        f32, i32 = torch.float32, torch.int32
        z = lambda *shape, dt: torch.empty(*shape, dtype=dt, device=self.dev)
        W = s.width
        self.logits = z(T1, s.E, dt=f32)
        self.topk_idx = z(T1, s.K, dt=i32) if not s.expert_choice else None
        self.topk_w = z(T1, W, dt=f32)
        self.lse = z(T1, dt=f32)
        self.counts = z(s.E, dt=i32)
        self.offsets = z(G + 1, dt=i32)
        self.slot_row = z(T1 * W, dt=i32)
        self.row_token = z(rows, dt=i32)
        self.row_slot = z(rows, dt=i32)
        self.n_dropped = z(4, dt=i32)
        self.x_perm = z(rows, s.D, dt=tdt)
        self.act = z(rows, 2 * s.F, dt=tdt)
        self.h = z(rows, s.F, dt=tdt)
        self.o_perm = z(rows, s.D, dt=tdt)
        self.y = z(T1, s.D, dt=tdt)
        self.losses = z(4, dt=f32)
        self.seq_loss = z(4, dt=f32)
        self.dlogits_aux = z(T1, s.E, dt=f32)
        self.ws = torch.empty(max(L.workspace_size(self.cfg), 256), dtype=torch.uint8,
                              device=self.dev)
        self.dx = z(T1, s.D, dt=tdt)
        self.dw_r = z(s.E, s.D, dt=f32)
        self.d_rbias = z(s.E, dt=f32)
        self.dw_gate = torch.empty_like(w_gate)
        self.dw_up = torch.empty_like(w_up)
        self.dw_down = torch.empty_like(w_down)
        self.d_logits = z(T1, s.E, dt=f32)
        self.noise_logits = z(T1, s.E, dt=f32) if w_noise is not None else None
        self.x = None
        # the losses and the bias step read only logits, indices and counts:
        # they run on a side stream (default priority) beside the expert FFN
        # and the combine, and the caller's stream waits for them at the end
        # of forward()
        self._side = torch.cuda.Stream(device=self.dev)
        self._fork = torch.cuda.Event()
        self._join = torch.cuda.Event()

    @property
    def use_aux(self) -> bool:
        return self.spec.score == L.MOE_SCORE_SOFTMAX and (self.spec.alpha != 0 or self.spec.zlam != 0)

    @property
    def use_seq(self) -> bool:
        return (self.spec.seq_len > 0 and self.spec.seq_alpha != 0
                and not self.spec.expert_choice)

    @property
    def has_dlogits(self) -> bool:
        return self.use_aux or self.use_seq

    def route(self, x, logits_given: bool = False, jitter=None, noise_eps=None):
        flags = L.MOE_ROUTE_LOGITS_GIVEN if logits_given else 0
        self.jitter = jitter
        if jitter is None and self.w_noise is None:
            L.moe_route(self.cfg, x, self.w_r, self.r_bias, self.sel_bias, self.logits,
                        self.topk_idx, self.topk_w, self.lse, flags)
        else:
            L.moe_route_ex(self.cfg, x, self.w_r, self.r_bias, self.sel_bias, jitter,
                           self.w_noise, noise_eps if self.w_noise is not None else None,
                           self.noise_logits, self.logits, self.topk_idx, self.topk_w, self.lse,
                           flags)

    def forward(self, x, logits_given: bool = False, jitter=None, noise_eps=None):
        """jitter / noise_eps: the step's random draws ([T][E] fp32) for the
        router-logit jitter and the noisy top-K selection (None: off)."""
        self.x = x
        if self.spec.expert_choice:
            self.jitter = None
            L.moe_route_expert_choice(self.cfg, x, self.w_r, self.r_bias, self.logits,
                                      self.topk_w, self.lse, self.counts, self.offsets,
                                      self.slot_row, self.row_token, self.row_slot, self.x_perm,
                                      self.ws, L.MOE_ROUTE_LOGITS_GIVEN if logits_given else 0)
        elif not logits_given and jitter is None and self.w_noise is None:
            # plain routing: route and permute in one call (fewer launches)
            self.jitter = None
            L.moe_route_permute(self.cfg, x, self.w_r, self.r_bias, self.sel_bias, self.logits,
                                self.topk_idx, self.topk_w, self.lse, self.counts, self.offsets,
                                self.slot_row, self.row_token, self.row_slot, self.n_dropped,
                                self.x_perm, self.ws)
        else:
            self.route(x, logits_given, jitter, noise_eps)
            L.moe_permute(self.cfg, self.topk_idx, x, self.counts, self.offsets, self.slot_row,
                          self.row_token, self.row_slot, self.n_dropped, self.x_perm, self.ws)
        main = torch.cuda.current_stream(self.dev)
        bias_step = (self.spec.bias_gamma != 0 and self.sel_bias is not None
                     and not self.spec.expert_choice)
        side = self.use_aux or self.use_seq or bias_step
        # MOE_SERIAL_STREAMS (measurement): the losses run on the main stream
        side_stream = main if os.environ.get("MOE_SERIAL_STREAMS") else self._side
        if side:
            self._fork.record(main)
            side_stream.wait_event(self._fork)
            if self.use_aux:
                L.aux_balance_loss(self.cfg, self.logits, self.counts, self.spec.alpha,
                                   self.spec.zlam, self.losses, self.dlogits_aux, self.ws,
                                   stream=side_stream)
            if self.use_seq:
                L.aux_seq_loss(self.cfg, self.logits, self.topk_idx, self.spec.seq_len,
                               self.spec.seq_alpha, self.seq_loss, self.dlogits_aux,
                               self.use_aux, self.ws, stream=side_stream)
            if bias_step:
                L.moe_bias_update(self.cfg, self.counts, self.spec.bias_gamma, self.sel_bias,
                                  stream=side_stream)
        L.moe_expert_ffn(self.cfg, x, self.x_perm, self.offsets, self.w_gate, self.w_up,
                         self.w_down, self.act, self.h, self.o_perm)
        L.moe_combine(self.cfg, self.o_perm, self.offsets, self.slot_row, self.topk_w, self.y)
        if side:
            self._join.record(side_stream)
            main.wait_event(self._join)
        return self.y

    def backward(self, dy, with_aux: bool | None = None):
        use = self.has_dlogits if with_aux is None else with_aux
        L.moe_backward_ex(self.cfg, self.x, self.w_r, self.logits, self.topk_idx, self.topk_w,
                          self.offsets, self.slot_row, self.x_perm, self.act, self.h,
                          self.o_perm, self.w_gate, self.w_up, self.w_down, dy,
                          self.dlogits_aux if use else None, self.jitter, self.dx, self.dw_r,
                          self.d_rbias, self.dw_gate, self.dw_up, self.dw_down, self.d_logits,
                          self.ws)
        return self.dx


class StepGraph:
    """One forward + backward of a ``MoELayer`` on fixed input buffers, captured
    once in a HIP graph and replayed: the same kernels, launched as one graph
    instead of one by one.  The library's side streams join the capture through
    their fork / join events.  ``x`` and ``dy`` are read in place at every
    replay, so refill them (``copy_``) to step on new data."""

    def __init__(self, layer: MoELayer, x, dy, with_aux: bool | None = None):
        self.layer, self.x, self.dy, self.with_aux = layer, x, dy, with_aux
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self._step()  # first launches (one-time set-up) outside the capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._step()

    def _step(self):
        self.layer.forward(self.x)
        self.layer.backward(self.dy, self.with_aux)

    def replay(self):
        self.graph.replay()
