"""Python wrapper of the CPU oracle (``oracle/moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` -- never by the product package.
It shares no code with the HIP library.  Inputs are numpy arrays: float64,
float32, or bf16 stored as raw ``uint16`` bit patterns; every value is widened
to double inside the C code.  Floating-point results come back as float64
(logits as float32, rounded once from a double sum).

Every function cites the page passage it implements in ``moe_oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

SOFTMAX, SIGMOID = 0, 1
GATE_A, GATE_B = 0, 1
_DT = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.float64): 2}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no contraction: the fp32 sigmoid key is a
    fixed IEEE operation sequence)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
             "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(C.Structure):
    _fields_ = [("T", C.c_int), ("D", C.c_int), ("E", C.c_int), ("K", C.c_int), ("F", C.c_int),
                ("lo", C.c_int), ("hi", C.c_int), ("n_shared", C.c_int), ("score", C.c_int),
                ("gating", C.c_int), ("cap", C.c_double), ("bug_mode", C.c_int)]


@dataclass
class Cfg:
    T: int
    D: int
    E: int
    K: int
    F: int
    lo: int = 0
    hi: int = -1           # -1: all experts local
    n_shared: int = 0
    score: int = SOFTMAX
    gating: int = GATE_B
    cap: float = 0.0       # <= 0: no capacity
    bug_mode: int = 0

    def c(self) -> _Cfg:
        hi = self.E if self.hi < 0 else self.hi
        return _Cfg(self.T, self.D, self.E, self.K, self.F, self.lo, hi, self.n_shared,
                    self.score, self.gating, float(self.cap), self.bug_mode)

    @property
    def n_local(self) -> int:
        return (self.E if self.hi < 0 else self.hi) - self.lo

    @property
    def groups(self) -> int:
        return self.n_local + self.n_shared


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB)
        P = C.c_void_p
        L.orc_set_threads.argtypes = [C.c_int]
        L.orc_get_threads.restype = C.c_int
        L.orc_exp32.argtypes = [C.c_float]
        L.orc_exp32.restype = C.c_float
        L.orc_sig32.argtypes = [C.c_float]
        L.orc_sig32.restype = C.c_float
        L.orc_capacity.argtypes = [P]
        L.orc_capacity.restype = C.c_long
        L.orc_logits.argtypes = [P, P, C.c_int, P, P, P, C.c_int, P]
        L.orc_logits64.argtypes = [P, P, C.c_int, P, P, P, C.c_int, P]
        L.orc_route.argtypes = [P, P, P, P, P, P, P]
        L.orc_dispatch.argtypes = [P, P, P, P, P, P, P, P]
        L.orc_forward.argtypes = [P, P, C.c_int, P, P, P, C.c_int, P, P, P, P, C.c_int, P]
        L.orc_expert_rows.argtypes = [P, P, C.c_int, P, P, P, C.c_int, P, P, C.c_int, P, P, P, P]
        L.orc_aux.argtypes = [P, P, P, C.c_double, C.c_double, P, P]
        L.orc_gate_grad.argtypes = [P, P, P, P, P, P]
        L.orc_bias_update.argtypes = [P, P, C.c_float, P]
        L.orc_ec_capacity.argtypes = [P]
        L.orc_ec_capacity.restype = C.c_long
        L.orc_route_ec.argtypes = [P, P, P, P, P, P, P]
        L.orc_route_ec.restype = C.c_int
        L.orc_seq_aux.argtypes = [P, P, P, C.c_int, C.c_double, P, P]
        L.orc_seq_aux.restype = C.c_int
        L.orc_group_wgrad_cols.argtypes = [P, P, C.c_int, P, P, P, C.c_int, P, P, P, P, C.c_int,
                                           P, C.c_int, P, P, P]
        L.orc_backward.argtypes = [P, P, C.c_int, P, P, P, P, C.c_int, P, P, P, P, P, C.c_int,
                                   P, P, P, C.c_int, P, P, P, P, P, P, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _arr(a, dtypes=(np.float32, np.uint16, np.float64)):
    a = np.ascontiguousarray(a)
    if a.dtype not in [np.dtype(d) for d in dtypes]:
        raise TypeError(f"unsupported dtype {a.dtype}")
    return a


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def threads() -> int:
    return int(lib().orc_get_threads())


def exp32(z: float) -> float:
    return float(lib().orc_exp32(float(z)))


def sig32(z: float) -> float:
    return float(lib().orc_sig32(float(z)))


def capacity(cfg: Cfg) -> int:
    c = cfg.c()
    return int(lib().orc_capacity(C.byref(c)))


def logits(cfg: Cfg, x, wr, rb=None, tok=None, exact: bool = False) -> np.ndarray:
    """O1: router logits for the listed tokens (all when tok is None): fp32,
    rounded once from the double sum; exact=True keeps the double sums."""
    x = _arr(x)
    wr = np.ascontiguousarray(wr, dtype=np.float64)   # exact widening of fp32
    rb = None if rb is None else np.ascontiguousarray(rb, dtype=np.float64)
    c = cfg.c()
    tk = None if tok is None else np.ascontiguousarray(tok, dtype=np.int32)
    n = cfg.T if tk is None else len(tk)
    out = np.empty((n, cfg.E), np.float64 if exact else np.float32)
    fn = lib().orc_logits64 if exact else lib().orc_logits
    fn(C.byref(c), _p(x), _DT[x.dtype], _p(wr), _p(rb), _p(tk), n, _p(out))
    return out


def route(cfg: Cfg, lg, selb=None):
    """O2-O4: top-K indices (pick order), gate weights, lse, full softmax."""
    lg = np.ascontiguousarray(lg, dtype=np.float64)
    assert lg.shape == (cfg.T, cfg.E)
    assert np.all(np.isfinite(lg)), "logits must be finite"
    selb = None if selb is None else np.ascontiguousarray(selb, dtype=np.float32)
    c = cfg.c()
    idx = np.empty((cfg.T, cfg.K), np.int32)
    w = np.empty((cfg.T, cfg.K), np.float64)
    lse = np.empty(cfg.T, np.float64)
    probs = np.empty((cfg.T, cfg.E), np.float64)
    lib().orc_route(C.byref(c), _p(lg), _p(selb), _p(idx), _p(w), _p(lse), _p(probs))
    return idx, w, lse, probs


def dispatch(cfg: Cfg, idx):
    """O5: counts, capacity, expert-major rows and the slot -> row map."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    c = cfg.c()
    G = cfg.groups
    nrows = cfg.T * cfg.K + cfg.n_shared * cfg.T
    counts = np.empty(cfg.E, np.int32)
    offsets = np.empty(G + 1, np.int32)
    slot_row = np.empty(cfg.T * cfg.K, np.int32)
    row_token = np.full(max(nrows, 1), -7, np.int32)
    row_slot = np.full(max(nrows, 1), -7, np.int32)
    nd = C.c_int(0)
    lib().orc_dispatch(C.byref(c), _p(idx), _p(counts), _p(offsets), _p(slot_row),
                       _p(row_token), _p(row_slot), C.byref(nd))
    n = int(offsets[-1])
    return dict(counts_all=counts, offsets=offsets, slot_row=slot_row,
                row_token=row_token[:n].copy(), row_slot=row_slot[:n].copy(),
                n_dropped=int(nd.value), capacity=capacity(cfg))


def forward(cfg: Cfg, x, wg, wu, wd, idx, w, slot_row, tok=None) -> np.ndarray:
    """O6-O7: layer output y for the listed tokens (float64)."""
    x, wg, wu, wd = _arr(x), _arr(wg), _arr(wu), _arr(wd)
    assert wg.dtype == wu.dtype == wd.dtype
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    slot_row = np.ascontiguousarray(slot_row, dtype=np.int32)
    tk = np.arange(cfg.T, dtype=np.int32) if tok is None else np.ascontiguousarray(tok, np.int32)
    y = np.empty((len(tk), cfg.D), np.float64)
    c = cfg.c()
    lib().orc_forward(C.byref(c), _p(x), _DT[x.dtype], _p(wg), _p(wu), _p(wd), _DT[wg.dtype],
                      _p(idx), _p(w), _p(slot_row), _p(tk), len(tk), _p(y))
    return y


def expert_rows(cfg: Cfg, x, wg, wu, wd, row_group, row_tok):
    """O6 per row: (a, b, h, o) of expert row_group[r] on token row_tok[r]."""
    x, wg, wu, wd = _arr(x), _arr(wg), _arr(wu), _arr(wd)
    rg = np.ascontiguousarray(row_group, dtype=np.int32)
    rt = np.ascontiguousarray(row_tok, dtype=np.int32)
    n = len(rg)
    a = np.empty((n, cfg.F)); b = np.empty((n, cfg.F)); h = np.empty((n, cfg.F))
    o = np.empty((n, cfg.D))
    c = cfg.c()
    lib().orc_expert_rows(C.byref(c), _p(x), _DT[x.dtype], _p(wg), _p(wu), _p(wd), _DT[wg.dtype],
                          _p(rg), _p(rt), n, _p(a), _p(b), _p(h), _p(o))
    return a, b, h, o


def aux(cfg: Cfg, lg, counts_all, alpha: float, zlam: float, want_grad: bool = True):
    """O8: (L_aux, L_z, mean lse^2) and d(L_aux + L_z)/d logits."""
    lg = np.ascontiguousarray(lg, dtype=np.float64)
    cnt = np.ascontiguousarray(counts_all, dtype=np.int32)
    losses = np.empty(3, np.float64)
    dl = np.empty((cfg.T, cfg.E), np.float64) if want_grad else None
    c = cfg.c()
    lib().orc_aux(C.byref(c), _p(lg), _p(cnt), float(alpha), float(zlam), _p(losses), _p(dl))
    return losses, dl


def bias_update(cfg: Cfg, counts_all, gamma: float, selb) -> np.ndarray:
    """Load-driven selection-bias step: returns the updated fp32 b (the input
    is not modified)."""
    cnt = np.ascontiguousarray(counts_all, dtype=np.int32)
    b = np.array(selb, dtype=np.float32, copy=True)
    c = cfg.c()
    lib().orc_bias_update(C.byref(c), _p(cnt), float(gamma), _p(b))
    return b


def ec_capacity(cfg: Cfg) -> int:
    """Expert-choice capacity: min(ceil(c T K / E), T), c = 1 when not given."""
    c = cfg.c()
    return int(lib().orc_ec_capacity(C.byref(c)))


def route_ec(cfg: Cfg, lg):
    """Expert-choice routing (softmax affinities; every local expert takes its
    C best tokens, equal keys to the lower token).  Returns a dict with
    slot_row [T,E] (row, -1 not taken, -2 not local), w [T,E] (p for every
    pair), row_token, offsets, lse, C, and the token-choice-shaped views
    idx [T,E] (identity) and cfg_w, the config with K = E and gating A under
    which forward() / backward() compute this layer."""
    lg = np.ascontiguousarray(lg, dtype=np.float64)
    c = cfg.c()
    T, E = cfg.T, cfg.E
    slot = np.empty((T, E), np.int32)
    w = np.empty((T, E), np.float64)
    Cap = ec_capacity(cfg)
    nrows = (cfg.n_local * Cap) + cfg.n_shared * T
    row_token = np.empty(max(nrows, 1), np.int32)
    offsets = np.empty(cfg.groups + 1, np.int32)
    lse = np.empty(T, np.float64)
    rc = lib().orc_route_ec(C.byref(c), _p(lg), _p(slot), _p(w), _p(row_token), _p(offsets),
                            _p(lse))
    if rc < 0:
        raise ValueError("expert choice needs softmax scoring")
    cw = Cfg(T=T, D=cfg.D, E=E, K=E, F=cfg.F, lo=cfg.lo, hi=cfg.hi, n_shared=cfg.n_shared,
             score=SOFTMAX, gating=0, cap=0.0)
    idx = np.tile(np.arange(E, dtype=np.int32), (T, 1))
    return dict(slot_row=slot, w=w, row_token=row_token[:nrows], offsets=offsets, lse=lse, C=rc,
                idx=idx, cfg_w=cw)


def route_noisy(cfg: Cfg, lg, jit=None, eps=None, nlg=None, selb=None, exact: bool = False):
    """Noisy top-K selection and router-logit jitter.

    [P3] ST-MoE: the router logits are multiplied by random factors u in
    [0.99, 1.01]:  s~ = s * u  (one binary32 multiply; in double when exact).
    [P3] KeepTopK / [P5] 8.6: the selection key adds input-dependent noise,
    H_e = s~_e + eps_e * softplus(n_e),  n = x W_noise,  eps ~ N(0, 1) per
    token and expert; evaluated in double and rounded once to binary32 (like
    the logits), then the usual top-K rounds (lowest index on ties).  [P3]
    states that the weights still come from the selected experts' noise-free
    logits (the noise only selects): weights, lse and probabilities are taken
    on s~ with the selected indices.  Noise is for softmax scoring only.
    Returns (idx, w, lse, probs, s~)."""
    s = np.asarray(lg, dtype=np.float64)
    if jit is not None:
        u = np.asarray(jit, dtype=np.float64)
        st = s * u if exact else (s.astype(np.float32) * u.astype(np.float32)).astype(np.float64)
    else:
        st = s
    if eps is None:
        idx, w, lse, probs = route(cfg, st, selb)
        return idx, w, lse, probs, st
    assert cfg.score == SOFTMAX, "noisy top-K is defined for softmax scoring"
    key = st + np.asarray(eps, np.float64) * np.logaddexp(0.0, np.asarray(nlg, np.float64))
    if not exact:
        key = key.astype(np.float32).astype(np.float64)
    idx = route(cfg, key)[0]
    m = st.max(1, keepdims=True)
    ex = np.exp(st - m)
    z = ex.sum(1, keepdims=True)
    probs = ex / z
    lse = (m + np.log(z))[:, 0]
    sel = np.take_along_axis(ex, idx.astype(np.int64), 1)
    w = sel / z if cfg.gating == 0 else sel / sel.sum(1, keepdims=True)
    return idx, w, lse, probs, st


def seq_aux(cfg: Cfg, lg, idx, seq_len: int, alpha: float, want_grad: bool = True):
    """Sequence-wise balance loss over sequences of seq_len tokens and its
    logit gradient [T,E] (f held constant)."""
    lg = np.ascontiguousarray(lg, dtype=np.float64)
    ix = np.ascontiguousarray(idx, dtype=np.int32)
    loss = np.zeros(1, np.float64)
    dl = np.empty((cfg.T, cfg.E), np.float64) if want_grad else None
    c = cfg.c()
    rc = lib().orc_seq_aux(C.byref(c), _p(lg), _p(ix), int(seq_len), float(alpha), _p(loss),
                           _p(dl))
    if rc != 0:
        raise ValueError(f"seq_len {seq_len} must divide T = {cfg.T}")
    return float(loss[0]), dl


def gate_grad(cfg: Cfg, lg, idx, w, dg) -> np.ndarray:
    """O11 alone: d loss / d logits [T,E] from d loss / d gate weights [T,K]."""
    lg = np.ascontiguousarray(lg, dtype=np.float64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    dg = np.ascontiguousarray(dg, dtype=np.float64)
    ds = np.empty((cfg.T, cfg.E))
    c = cfg.c()
    lib().orc_gate_grad(C.byref(c), _p(lg), _p(idx), _p(w), _p(dg), _p(ds))
    return ds


def backward(cfg: Cfg, x, wr, wg, wu, wd, lg, idx, w, slot_row, dy, tok=None, dlx=None,
             fsel=None, want_wgrad=True, want_rgrad=True, jit=None):
    """O9-O12.  dy rows belong to the listed tokens (all when tok is None);
    every other token has dy = 0.  Returns dx and ds for the listed tokens,
    dW_r, d r_b and the expert weight gradients on the F-columns fsel."""
    x, wg, wu, wd = _arr(x), _arr(wg), _arr(wu), _arr(wd)
    assert wg.dtype == wu.dtype == wd.dtype
    wr = np.ascontiguousarray(wr, dtype=np.float64)
    lg = np.ascontiguousarray(lg, dtype=np.float64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    slot_row = np.ascontiguousarray(slot_row, dtype=np.int32)
    tk = np.arange(cfg.T, dtype=np.int32) if tok is None else np.ascontiguousarray(tok, np.int32)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    assert dy.shape == (len(tk), cfg.D)
    dlx = None if dlx is None else np.ascontiguousarray(dlx, dtype=np.float64)
    jt = None if jit is None else np.ascontiguousarray(jit, dtype=np.float32)
    fs = None if fsel is None else np.ascontiguousarray(fsel, dtype=np.int32)
    nf = cfg.F if fs is None else len(fs)
    G = cfg.groups
    dx = np.empty((len(tk), cfg.D)); ds = np.empty((len(tk), cfg.E))
    dwr = np.empty((cfg.E, cfg.D)) if want_rgrad else None
    drb = np.empty(cfg.E) if want_rgrad else None
    dwg = np.empty((G, cfg.D, nf)) if want_wgrad else None
    dwu = np.empty((G, cfg.D, nf)) if want_wgrad else None
    dwd = np.empty((G, nf, cfg.D)) if want_wgrad else None
    c = cfg.c()
    lib().orc_backward(C.byref(c), _p(x), _DT[x.dtype], _p(wr), _p(wg), _p(wu), _p(wd),
                       _DT[wg.dtype], _p(lg), _p(idx), _p(w), _p(slot_row), _p(tk), len(tk),
                       _p(dy), _p(dlx), _p(fs), nf, _p(dx), _p(ds), _p(dwr), _p(drb),
                       _p(dwg), _p(dwu), _p(dwd), _p(jt))
    return dict(dx=dx, ds=ds, dwr=dwr, drb=drb, dwg=dwg, dwu=dwu, dwd=dwd)


def group_wgrad_cols(cfg: Cfg, x, wg, wu, wd, idx, w, slot_row, dy, g: int, fsel):
    """O10 on F-columns fsel for group g from every row of the group, with the
    dense upstream gradient dy [T][D]: (dW_gate[g][:, fsel], dW_up[g][:, fsel],
    dW_down[g][fsel, :]).  Routed group g is expert lo + g (kept local slots,
    weight g_{t,k}); g >= n_local is the shared expert (every token, weight 1)."""
    x, wg, wu, wd = _arr(x), _arr(wg), _arr(wu), _arr(wd)
    assert wg.dtype == wu.dtype == wd.dtype
    assert 0 <= g < cfg.groups
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    slot_row = np.ascontiguousarray(slot_row, dtype=np.int32)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    assert dy.shape == (cfg.T, cfg.D)
    fs = np.ascontiguousarray(fsel, dtype=np.int32)
    nf = len(fs)
    dwg = np.empty((cfg.D, nf)); dwu = np.empty((cfg.D, nf)); dwd = np.empty((nf, cfg.D))
    c = cfg.c()
    lib().orc_group_wgrad_cols(C.byref(c), _p(x), _DT[x.dtype], _p(wg), _p(wu), _p(wd),
                               _DT[wg.dtype], _p(idx), _p(w), _p(slot_row), _p(dy), int(g),
                               _p(fs), nf, _p(dwg), _p(dwu), _p(dwd))
    return dwg, dwu, dwd


def layer(cfg: Cfg, x, wr, wg, wu, wd, dy=None, rb=None, selb=None, alpha=0.0, zlam=0.0,
          exact_logits=False):
    """Convenience: the whole layer (O1-O12) on all tokens, for small sizes."""
    lg = logits(cfg, x, wr, rb, exact=exact_logits)
    idx, w, lse, probs = route(cfg, lg, selb)
    dsp = dispatch(cfg, idx)
    y = forward(cfg, x, wg, wu, wd, idx, w, dsp["slot_row"])
    out = dict(logits=lg, idx=idx, w=w, lse=lse, probs=probs, y=y, **dsp)
    if cfg.score == SOFTMAX:
        losses, dl = aux(cfg, lg, dsp["counts_all"], alpha, zlam)
        out.update(losses=losses, dlogits_aux=dl)
    else:
        dl = None
    if dy is not None:
        use_dl = dl if (alpha != 0.0 or zlam != 0.0) else None
        out.update(backward(cfg, x, wr, wg, wu, wd, lg, idx, w, dsp["slot_row"], dy, dlx=use_dl))
    return out
