"""Seeded synthetic inputs for the MoE layer workloads.

This module holds no arithmetic of the layer itself: it only names the
workload shapes and draws seeded random tensors with the distributions of the
layer configurations (tokens x ~ N(0,1), router weight ~ N(0, 0.02), expert
weights ~ N(0, 1/sqrt(D)), upstream gradient ~ N(0,1); standard deviations).
Both the HIP path (tests, benchmark) and the CPU oracle receive the same
arrays from here.

Two seeded back-ends:
* ``host``: numpy PCG64 from ``SeedSequence(seed).spawn``, one child per
  tensor and one child per expert matrix, fp64 normals -> fp32 -> bf16 (round
  to nearest even).  Used for every size the oracle checks densely.
* ``device``: torch's on-device Philox generator, one seed per tensor and per
  expert matrix (derived from the same SeedSequence), used for the full-size
  workloads whose weights (up to 22.6 GB) would take minutes to draw on the
  host.  The oracle then reads back the rows / experts it samples.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

SOFTMAX, SIGMOID = 0, 1
GATE_A, GATE_B = 0, 1
F32, BF16 = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    D: int
    E: int
    K: int
    F: int
    dtype: int = BF16
    lo: int = 0
    hi: int = -1               # -1: every expert local
    n_shared: int = 0
    score: int = SOFTMAX
    gating: int = GATE_B
    cap: float = 0.0           # capacity factor (<= 0: none)
    hot_bias: float = 0.0      # router bias on expert 0 (hotspot)
    sel_bias: float = 0.0      # selection bias b_e ~ U(-sel_bias, sel_bias)
    alpha: float = 0.0         # Switch balance-loss coefficient
    zlam: float = 0.0          # router z-loss coefficient
    seed: int = 0
    note: str = ""

    @property
    def local_hi(self) -> int:
        return self.E if self.hi < 0 else self.hi

    @property
    def n_local(self) -> int:
        return self.local_hi - self.lo

    @property
    def groups(self) -> int:
        return self.n_local + self.n_shared

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five layer configurations (shapes, dtypes, routing variants).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", T=256, D=64, E=4, K=2, F=128, dtype=F32,
                          gating=GATE_B, note="tiny fp32 layer, softmax/B, dropless"),
    "minimind": Workload("minimind", T=4096, D=768, E=4, K=2, F=2048, gating=GATE_B,
                         alpha=5e-4, note="MiniMind-like 16x256 tokens; K in {1,2}, A/B"),
    "olmoe_share": Workload("olmoe_share", T=8192, D=2048, E=64, K=8, F=1024, lo=0, hi=32,
                            gating=GATE_B, note="OLMoE-like: experts 0-31 local, 32-63 sentinel"),
    "mixtral_cap": Workload("mixtral_cap", T=16384, D=4096, E=8, K=2, F=14336, gating=GATE_B,
                            cap=1.25, hot_bias=2.0, zlam=1e-3,
                            note="Mixtral-like, capacity 1.25, hotspot bias +2 on expert 0"),
    "deepseek_v3": Workload("deepseek_v3", T=8192, D=7168, E=256, K=8, F=2048, n_shared=1,
                            score=SIGMOID, gating=GATE_B, sel_bias=0.1,
                            note="DeepSeek-V3-style sigmoid + selection bias, 1 shared expert"),
}


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _cast(a32: np.ndarray, dtype: int) -> np.ndarray:
    return bf16_bits(a32) if dtype == BF16 else np.ascontiguousarray(a32, np.float32)


@dataclass
class HostInputs:
    """Arrays in their storage dtype (bf16 as uint16 bit patterns)."""
    wl: Workload
    x: np.ndarray
    wr: np.ndarray
    rb: np.ndarray | None
    selb: np.ndarray | None
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray
    dy: np.ndarray
    extra: dict = field(default_factory=dict)


def _children(seed: int, n: int):
    return np.random.SeedSequence(seed).spawn(n)


def host_inputs(wl: Workload, seed: int | None = None) -> HostInputs:
    seed = wl.seed if seed is None else seed
    G = wl.groups
    ch = _children(seed, 6)
    x = np.random.Generator(np.random.PCG64(ch[0])).standard_normal((wl.T, wl.D))
    wr = np.random.Generator(np.random.PCG64(ch[1])).standard_normal((wl.E, wl.D)) * 0.02
    dy = np.random.Generator(np.random.PCG64(ch[2])).standard_normal((wl.T, wl.D))
    rb = None
    if wl.hot_bias:
        rb = np.zeros(wl.E, np.float32)
        rb[0] = wl.hot_bias
    selb = None
    if wl.sel_bias:
        selb = np.random.Generator(np.random.PCG64(ch[3])).uniform(
            -wl.sel_bias, wl.sel_bias, wl.E).astype(np.float32)
    std = 1.0 / np.sqrt(wl.D)
    wch = ch[4].spawn(3 * G)
    mats = []
    for m, shape in enumerate([(wl.D, wl.F), (wl.D, wl.F), (wl.F, wl.D)]):
        arr = np.empty((G,) + shape, np.uint16 if wl.dtype == BF16 else np.float32)
        for g in range(G):
            v = np.random.Generator(np.random.PCG64(wch[m * G + g])).standard_normal(shape) * std
            arr[g] = _cast(v.astype(np.float32), wl.dtype)
        mats.append(arr)
    return HostInputs(wl, _cast(x.astype(np.float32), wl.dtype), wr.astype(np.float32), rb, selb,
                      mats[0], mats[1], mats[2], _cast(dy.astype(np.float32), wl.dtype))


def device_inputs(wl: Workload, device="cuda", seed: int | None = None):
    """Full-size inputs drawn on the GPU with torch's seeded Philox generator.

    Returns a dict of torch tensors (bf16 / fp32 storage dtypes)."""
    import torch

    seed = wl.seed if seed is None else seed
    G = wl.groups
    ss = np.random.SeedSequence(seed)
    seeds = [int(s) for s in ss.generate_state(6 + 3 * G, dtype=np.uint32)]
    tdt = torch.bfloat16 if wl.dtype == BF16 else torch.float32

    def normal(shape, s, std=1.0, dtype=tdt):
        g = torch.Generator(device=device)
        g.manual_seed(s)
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t.to(dtype)

    out = {}
    out["x"] = normal((wl.T, wl.D), seeds[0])
    out["wr"] = normal((wl.E, wl.D), seeds[1], 0.02, torch.float32)
    out["dy"] = normal((wl.T, wl.D), seeds[2])
    out["rb"] = None
    if wl.hot_bias:
        rb = torch.zeros(wl.E, device=device, dtype=torch.float32)
        rb[0] = wl.hot_bias
        out["rb"] = rb
    out["selb"] = None
    if wl.sel_bias:
        g = torch.Generator(device=device)
        g.manual_seed(seeds[3])
        out["selb"] = (torch.rand(wl.E, generator=g, device=device) * 2 - 1) * wl.sel_bias
    std = 1.0 / float(np.sqrt(wl.D))
    for m, (name, shape) in enumerate([("wg", (wl.D, wl.F)), ("wu", (wl.D, wl.F)),
                                       ("wd", (wl.F, wl.D))]):
        t = torch.empty((G,) + shape, device=device, dtype=tdt)
        for gi in range(G):
            t[gi] = normal(shape, seeds[6 + m * G + gi], std)
        out[name] = t
    return out


def random_logits(T: int, E: int, seed: int, scale: float = 1.0, ties: bool = False) -> np.ndarray:
    """Seeded fp32 logits for routing tests; ties=True quantises them so that
    equal keys are frequent (exercises the lowest-index tie rule)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    lg = rng.standard_normal((T, E)) * scale
    if ties:
        lg = np.round(lg * 2) / 2
    return lg.astype(np.float32)


def routing_noise(wl: Workload, seed: int | None = None, device=None):
    """The random draws of the router-noise variants, as inputs:
    jitter u ~ U[0.99, 1.01] [T][E] (ST-MoE logit jitter), eps ~ N(0, 1) [T][E]
    (noisy top-K, one draw per token and expert) and a noise router
    W_noise ~ N(0, 0.02) [E][D] (same scale as W_r), all fp32.  numpy arrays
    (device None) or torch tensors on `device` (seeded Philox)."""
    seed = (wl.seed if seed is None else seed) + 7919
    if device is None:
        ch = np.random.SeedSequence(seed).spawn(3)
        u = np.random.Generator(np.random.PCG64(ch[0])).uniform(0.99, 1.01, (wl.T, wl.E))
        eps = np.random.Generator(np.random.PCG64(ch[1])).standard_normal((wl.T, wl.E))
        wn = np.random.Generator(np.random.PCG64(ch[2])).standard_normal((wl.E, wl.D)) * 0.02
        return u.astype(np.float32), eps.astype(np.float32), wn.astype(np.float32)
    import torch
    seeds = [int(s) for s in np.random.SeedSequence(seed).generate_state(3, dtype=np.uint32)]
    gens = []
    for s in seeds:
        g = torch.Generator(device=device)
        g.manual_seed(s)
        gens.append(g)
    u = torch.rand(wl.T, wl.E, generator=gens[0], device=device) * 0.02 + 0.99
    eps = torch.randn(wl.T, wl.E, generator=gens[1], device=device)
    wn = torch.randn(wl.E, wl.D, generator=gens[2], device=device) * 0.02
    return u, eps, wn
