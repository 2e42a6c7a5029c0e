"""Pins of the CPU oracle against what the pages and the mathematics fix.

These run without a GPU.  Each test names the passage it pins.  They are
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign or
index, a transposed operand, a wrong normalisation) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest

from mixture_experts_layer_23_amd import synthetic as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def tiny_inputs(rng, T, D, E, F, G):
    x = rng.standard_normal((T, D))
    wr = rng.standard_normal((E, D)) * 0.5
    wg = rng.standard_normal((G, D, F)) / math.sqrt(D)
    wu = rng.standard_normal((G, D, F)) / math.sqrt(D)
    wd = rng.standard_normal((G, F, D)) / math.sqrt(F)
    dy = rng.standard_normal((T, D))
    return x, wr, wg, wu, wd, dy


# --------------------------------------------------------------------------
# P1 gating worked example (course notes 8.2)
# --------------------------------------------------------------------------
def test_gating_worked_example(orc):
    g = gold("gating_example.json")
    lg = np.log(np.array([g["probs"]], np.float64)).astype(np.float32)
    for gating, key in [(orc.GATE_A, "gate_A"), (orc.GATE_B, "gate_B")]:
        cfg = orc.Cfg(T=1, D=1, E=4, K=g["K"], F=8, gating=gating)
        idx, w, lse, probs = orc.route(cfg, lg)
        assert idx[0].tolist() == g["topk"]
        np.testing.assert_allclose(w[0], g[key], rtol=1e-6)
        np.testing.assert_allclose(probs[0], g["probs"], rtol=1e-6)
        # lse of log-probabilities that sum to one is zero
        assert abs(lse[0]) < 1e-6


def test_gating_B_equals_keeptopk_softmax(orc):
    """KeepTopK (tutorial, Load Balancing: KeepTopK): softmax over logits with
    the non-top-K set to -inf gives the renormalised weights of gating B."""
    lg = S.random_logits(64, 9, seed=3, scale=2.0)
    cfg = orc.Cfg(T=64, D=1, E=9, K=3, F=8, gating=orc.GATE_B)
    idx, w, _, _ = orc.route(cfg, lg)
    for t in range(64):
        v = np.full(9, -np.inf)
        v[idx[t]] = lg[t, idx[t]].astype(np.float64)
        e = np.exp(v - v.max())
        np.testing.assert_allclose(w[t], (e / e.sum())[idx[t]], rtol=1e-12)


# --------------------------------------------------------------------------
# top-K selection: brute force, tie rule, sigmoid key
# --------------------------------------------------------------------------
def test_topk_brute_force_with_ties(orc):
    lg = S.random_logits(300, 7, seed=11, ties=True)
    assert (lg[:, :, None] == lg[:, None, :]).sum() > 300 * 7  # many equal keys
    for K in (1, 2, 3, 7):
        cfg = orc.Cfg(T=300, D=1, E=7, K=K, F=8)
        idx, _, _, _ = orc.route(cfg, lg)
        for t in range(300):
            # sort by (-key, index): descending key, lowest index first on ties
            want = sorted(range(7), key=lambda e: (-float(lg[t, e]), e))[:K]
            assert idx[t].tolist() == want


def test_signed_zero_is_a_tie(orc):
    lg = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32)
    cfg = orc.Cfg(T=2, D=1, E=3, K=1, F=8)
    idx, _, _, _ = orc.route(cfg, lg)
    assert idx[:, 0].tolist() == [0, 0]


def test_exp32_sig32_accuracy_and_order(orc):
    zs = np.linspace(-30, 30, 4001, dtype=np.float32)
    ex = np.array([orc.exp32(float(z)) for z in zs], np.float32)
    ref = np.exp(zs.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(ex - ref) / ulp) <= 2.0
    sg = np.array([orc.sig32(float(z)) for z in zs], np.float32)
    ref = 1.0 / (1.0 + np.exp(-zs.astype(np.float64)))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(sg - ref) / ulp) <= 2.0
    assert np.all(np.diff(sg.astype(np.float64)) >= 0)
    assert orc.sig32(0.0) == 0.5
    # clamp: beyond +-87 the key saturates instead of overflowing
    assert orc.sig32(200.0) == 1.0 and 0.0 < orc.sig32(-200.0) < 1e-37


def test_sigmoid_selection_uses_bias_weights_do_not(orc):
    """Course notes 8.6: select on s_e + b_e, aggregate on the raw scores."""
    T, E, K = 50, 16, 4
    lg = S.random_logits(T, E, seed=5)
    b = np.random.default_rng(1).uniform(-0.3, 0.3, E).astype(np.float32)
    for gating in (orc.GATE_A, orc.GATE_B):
        cfg = orc.Cfg(T=T, D=1, E=E, K=K, F=8, score=orc.SIGMOID, gating=gating)
        idx, w, _, _ = orc.route(cfg, lg, b)
        for t in range(T):
            key = [np.float32(orc.sig32(float(lg[t, e]))) + b[e] for e in range(E)]
            want = sorted(range(E), key=lambda e: (-float(key[e]), e))[:K]
            assert idx[t].tolist() == want
            sg = 1.0 / (1.0 + np.exp(-lg[t, idx[t]].astype(np.float64)))
            np.testing.assert_allclose(w[t], sg if gating == orc.GATE_A else sg / sg.sum(),
                                       rtol=1e-12)


# --------------------------------------------------------------------------
# P2 Switch balance loss (course notes 8.5) and P6 (MiniMind aux floor)
# --------------------------------------------------------------------------
def _switch_case(orc):
    g = gold("switch_loss_example.json")
    p0 = np.array([0.7, 0.7, 0.7, 0.3])
    lg = np.log(np.stack([p0, 1 - p0], 1))
    cfg = orc.Cfg(T=4, D=1, E=2, K=1, F=8)
    return g, cfg, lg


def test_switch_loss_worked_example(orc):
    g, cfg, lg = _switch_case(orc)
    idx, _, _, probs = orc.route(cfg, lg)
    counts = np.bincount(idx.ravel(), minlength=2)
    np.testing.assert_allclose(counts / 4, g["f"])
    np.testing.assert_allclose(probs.mean(0), g["P"], rtol=1e-12)
    losses, _ = orc.aux(cfg, lg, counts, g["alpha"], 0.0)
    assert abs(losses[0] - g["L"]) < 1e-12


def test_switch_loss_gradient_closed_form(orc):
    """dL/dp_{t,e} = alpha*E*f_e/T with f held constant, chained through the
    softmax Jacobian by hand and by finite differences on the logits."""
    g, cfg, lg = _switch_case(orc)
    idx, _, _, probs = orc.route(cfg, lg)
    counts = np.bincount(idx.ravel(), minlength=2)
    _, dl = orc.aux(cfg, lg, counts, g["alpha"], 0.0)
    dLdp = g["alpha"] * 2 * np.array(g["f"]) / 4
    np.testing.assert_allclose(dLdp, [0.00375, 0.00125])
    for t in range(4):
        p = probs[t]
        J = np.diag(p) - np.outer(p, p)          # d p / d s
        np.testing.assert_allclose(dl[t], J.T @ dLdp, atol=1e-15)
    h = 1e-6
    for t in range(4):
        for e in range(2):
            lp, lm = lg.copy(), lg.copy()
            lp[t, e] += h
            lm[t, e] -= h
            fd = (orc.aux(cfg, lp, counts, g["alpha"], 0.0)[0][0]
                  - orc.aux(cfg, lm, counts, g["alpha"], 0.0)[0][0]) / (2 * h)
            assert abs(fd - dl[t, e]) < 1e-9


def test_switch_loss_limits(orc):
    E, T, alpha = 4, 64, 0.01
    cfg = orc.Cfg(T=T, D=1, E=E, K=1, F=8)
    lg = np.zeros((T, E))
    losses, _ = orc.aux(cfg, lg, np.full(E, T // E), alpha, 0.0)
    assert abs(losses[0] - alpha) < 1e-15           # uniform: f = P = 1/E
    lg = np.full((T, E), -60.0)
    lg[:, 2] = 60.0
    losses, _ = orc.aux(cfg, lg, np.array([0, 0, T, 0]), alpha, 0.0)
    assert abs(losses[0] - alpha * E) < 1e-12       # collapse: ~ alpha*E


def test_minimind_aux_floor(orc):
    """MiniMind issue section 1: floor 0.004000 over 8 layers = 8 * alpha, i.e.
    a per-layer minimum of alpha at f = P = 1/E (K = 1)."""
    g = gold("minimind_aux_floor.json")
    cfg = orc.Cfg(T=256, D=1, E=g["E"], K=g["K"], F=8)
    losses, _ = orc.aux(cfg, np.zeros((256, 4)), np.full(4, 64), g["alpha"], 0.0)
    assert abs(g["layers"] * losses[0] - g["aux_floor_total"]) < 1e-15


def test_z_loss_definition_and_gradient(orc):
    """Tutorial, ST-MoE: L_z = lambda * mean_t (log sum_e exp s_te)^2."""
    T, E, lam = 6, 5, 0.3
    lg = S.random_logits(T, E, seed=2, scale=3.0).astype(np.float64)
    cfg = orc.Cfg(T=T, D=1, E=E, K=2, F=8)
    cnt = np.array([3, 2, 4, 1, 2])
    losses, dl = orc.aux(cfg, lg, cnt, 0.0, lam)
    lse = np.log(np.exp(lg).sum(1))
    assert abs(losses[1] - lam * np.mean(lse ** 2)) < 1e-12
    assert abs(losses[2] - np.mean(lse ** 2)) < 1e-12
    h = 1e-6
    for t in range(T):
        for e in range(E):
            lp, lm = lg.copy(), lg.copy()
            lp[t, e] += h
            lm[t, e] -= h
            fd = (orc.aux(cfg, lp, cnt, 0.0, lam)[0][1] - orc.aux(cfg, lm, cnt, 0.0, lam)[0][1]) / (2 * h)
            assert abs(fd - dl[t, e]) < 1e-8


def test_z_loss_equal_logits_closed_form(orc):
    """Tutorial, ST-MoE (z-loss on the log-sum-exp of the router logits):
    with all E logits of a token equal to c, lse = c + ln E, so the z-loss is
    lambda (c + ln E)^2 and its logit gradient lambda (2/T) lse / E in every
    entry (p = 1/E).  A dropped square, a missing ln E, a sum instead of a
    mean over tokens or a wrong gradient factor fails here."""
    T, lam = 7, 0.25
    for E in (2, 5, 64):
        for c in (-3.0, 0.0, 1.7):
            cfg = orc.Cfg(T=T, D=1, E=E, K=1, F=8)
            lg = np.full((T, E), c)
            cnt = np.zeros(E, np.int32)
            cnt[0] = T
            losses, dl = orc.aux(cfg, lg, cnt, 0.0, lam)
            want = (c + math.log(E)) ** 2
            assert abs(losses[2] - want) <= 1e-13 * max(1.0, want)
            assert abs(losses[1] - lam * want) <= 1e-13 * max(1.0, want)
            np.testing.assert_allclose(dl, lam * (2.0 / T) * (c + math.log(E)) / E,
                                       rtol=1e-12, atol=1e-15)


def test_z_loss_hand_worked_example(orc):
    """Two tokens whose exp-logits are small integers: the log-sum-exps are
    exactly 2 ln 2 and 3 ln 2 (tests/golden/z_loss_example.json)."""
    g = gold("z_loss_example.json")
    ex = np.array(g["exp_logits"])
    lg = np.log(ex)
    T, E = ex.shape
    cfg = orc.Cfg(T=T, D=1, E=E, K=1, F=8)
    losses, dl = orc.aux(cfg, lg, np.array([T, 0, 0]), 0.0, g["lambda"])
    assert abs(losses[2] - g["mean_lse2"]) < 1e-12
    assert abs(losses[1] - g["z_loss"]) < 1e-15
    lse = np.array([2.0, 3.0]) * math.log(2.0)
    p = np.array([0.25, 0.25, 0.5])
    np.testing.assert_allclose(dl, g["lambda"] * (2.0 / T) * lse[:, None] * p[None, :],
                               rtol=1e-12)


@pytest.mark.parametrize("K", [2, 4])
def test_switch_loss_limits_top_k(orc, K):
    """Course notes 8.5 state the balance loss's limits: alpha when load and
    probability are uniform, alpha*E when everything collapses.  For K > 1
    the uniform limit holds only with f_e normalised by the T*K slots (the
    page warns the normaliser varies); with f normalised by T alone it would
    read K*alpha.  Collapse onto K experts (every token picks the same K, the
    probability split evenly over them) then gives alpha*E/K."""
    E, T, alpha = 8, 64, 0.01
    cfg = orc.Cfg(T=T, D=1, E=E, K=K, F=8)
    losses, _ = orc.aux(cfg, np.zeros((T, E)), np.full(E, T * K // E), alpha, 0.0)
    assert abs(losses[0] - alpha) < 1e-15
    lg = np.full((T, E), -80.0)
    lg[:, :K] = 0.0
    cnt = np.zeros(E, np.int32)
    cnt[:K] = T
    losses, _ = orc.aux(cfg, lg, cnt, alpha, 0.0)
    assert abs(losses[0] - alpha * E / K) < 1e-12
    # the routing the oracle itself picks on these logits gives these counts
    idx, _, _, _ = orc.route(cfg, lg)
    assert np.array_equal(np.bincount(idx.ravel(), minlength=E), cnt)


def test_group_wgrad_columns_equal_full_backward(orc):
    """The column-restricted weight gradient of one group (used at full size,
    where the full backward is too slow) equals the columns of the full
    backward with a dense upstream gradient, for routed groups with drops and
    sentinels around them and for the shared expert."""
    rng = np.random.default_rng(17)
    T, D, E, K, F = 40, 16, 6, 2, 24
    cfg = orc.Cfg(T=T, D=D, E=E, K=K, F=F, lo=1, hi=5, n_shared=1, cap=0.9)
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, E, F, cfg.groups)
    lg = orc.logits(cfg, x, wr)
    idx, w, _, _ = orc.route(cfg, lg)
    d = orc.dispatch(cfg, idx)
    assert d["n_dropped"] > 0 and np.any(d["slot_row"] == -2)
    fsel = np.array([0, 5, 11, 23])
    full = orc.backward(cfg, x, wr, wg, wu, wd, lg, idx, w, d["slot_row"], dy, fsel=fsel)
    for g in range(cfg.groups):
        a, b, c = orc.group_wgrad_cols(cfg, x, wg, wu, wd, idx, w, d["slot_row"], dy, g, fsel)
        np.testing.assert_allclose(a, full["dwg"][g], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(b, full["dwu"][g], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(c, full["dwd"][g], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# P5 capacity and drops (course lab printout) + P10 integer invariants
# --------------------------------------------------------------------------
def test_capacity_lab_numbers(orc):
    g = gold("capacity_lab.json")
    T, E, K = g["T"], g["E"], g["K"]
    second = np.array([1] * 107 + [2] * 60 + [3] * 89)
    idx = np.stack([np.zeros(T, int), second], 1)
    cfg = orc.Cfg(T=T, D=8, E=E, K=K, F=8, cap=1.1)
    d = orc.dispatch(cfg, idx)
    assert d["capacity"] == g["capacity"]
    assert d["counts_all"].tolist() == g["loads_hotspot"]
    assert d["n_dropped"] == g["dropped_hotspot"]
    # the dropped assignments are expert 0's, tokens 141..255 (token order)
    dropped = np.nonzero(d["slot_row"] == -1)[0]
    assert dropped.tolist() == [t * K for t in range(141, 256)]
    # no hotspot: loads [139,137,117,119] -> nothing dropped.  Build a routing
    # with exactly these loads: each token takes the two experts with the most
    # remaining demand.
    loads = g["loads_no_hotspot"]
    need = list(loads)
    rows = []
    for t in range(T):
        a = int(np.argmax(need))
        need[a] -= 1
        b = int(np.argmax([n if e != a else -1 for e, n in enumerate(need)]))
        need[b] -= 1
        rows.append((a, b))
    assert need == [0, 0, 0, 0]
    d = orc.dispatch(cfg, np.array(rows))
    assert d["counts_all"].tolist() == loads and d["n_dropped"] == g["dropped_no_hotspot"]


def _brute_dispatch(idx, E, lo, hi, C, n_shared):
    T, K = idx.shape
    slots = [(t, k, int(idx[t, k])) for t in range(T) for k in range(K)]
    counts = [sum(1 for s in slots if s[2] == e) for e in range(E)]
    local = sorted([s for s in slots if lo <= s[2] < hi], key=lambda s: (s[2], s[0]))
    slot_row = {}
    pos = {}
    rows = []
    for t, k, e in local:
        p = pos.get(e, 0)
        pos[e] = p + 1
        if C >= 0 and p >= C:
            slot_row[(t, k)] = -1
        else:
            slot_row[(t, k)] = len(rows)
            rows.append((t, t * K + k))
    for _ in range(n_shared):
        rows += [(t, -1) for t in range(T)]
    sr = np.array([slot_row.get((t, k), -2) for t in range(T) for k in range(K)])
    return counts, sr, rows


@pytest.mark.parametrize("T,E,K,lo,hi,cap,ns", [
    (37, 5, 2, 0, 5, 0.0, 0), (64, 8, 3, 2, 6, 1.0, 0), (50, 4, 4, 0, 4, 0.5, 1),
    (1, 3, 1, 1, 2, 1.0, 0), (0, 4, 2, 0, 4, 1.25, 1), (40, 6, 2, 6, 6, 0.0, 0),
    (33, 64, 8, 0, 32, 1.0, 0)])
def test_dispatch_brute_force_and_invariants(orc, T, E, K, lo, hi, cap, ns):
    rng = np.random.default_rng(T * 131 + E)
    idx = np.array([rng.permutation(E)[:K] for _ in range(T)]).reshape(T, K)
    cfg = orc.Cfg(T=T, D=8, E=E, K=K, F=8, lo=lo, hi=hi, cap=cap, n_shared=ns)
    d = orc.dispatch(cfg, idx)
    C = d["capacity"]
    counts, sr, rows = _brute_dispatch(idx, E, lo, hi, C, ns)
    assert d["counts_all"].tolist() == counts
    assert d["slot_row"].tolist() == sr.tolist()
    assert d["row_token"].tolist() == [r[0] for r in rows]
    assert d["row_slot"].tolist() == [r[1] for r in rows]
    # invariants
    assert sum(counts) == T * K
    kept = np.diff(d["offsets"])[: hi - lo]
    for j in range(hi - lo):
        assert kept[j] == (min(counts[lo + j], C) if C >= 0 else counts[lo + j])
    nsent = int((d["slot_row"] == -2).sum())
    assert kept.sum() + d["n_dropped"] + nsent == T * K
    assert d["offsets"][-1] == kept.sum() + ns * T


# --------------------------------------------------------------------------
# P9 special cases that reduce to textbook routines (numpy)
# --------------------------------------------------------------------------
def _silu(a):
    return a / (1 + np.exp(-a))


def _ffn(x, wg, wu, wd):
    return (_silu(x @ wg) * (x @ wu)) @ wd


def test_single_expert_is_dense_swiglu(orc):
    rng = np.random.default_rng(0)
    T, D, F = 9, 12, 16
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, 1, F, 1)
    for gating in (orc.GATE_A, orc.GATE_B):
        cfg = orc.Cfg(T=T, D=D, E=1, K=1, F=F, gating=gating)
        out = orc.layer(cfg, x, wr, wg, wu, wd)
        np.testing.assert_allclose(out["y"], _ffn(x, wg[0], wu[0], wd[0]), rtol=1e-12, atol=1e-12)


def test_k_equals_e_is_dense_soft_mixture(orc):
    """Tutorial, Router/Gating Network: y = sum_i G(x)_i E_i(x) with
    G = softmax(x W_g) when every expert is selected (gating B)."""
    rng = np.random.default_rng(1)
    T, D, E, F = 11, 10, 5, 12
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, E, F, E)
    cfg = orc.Cfg(T=T, D=D, E=E, K=E, F=F, gating=orc.GATE_B)
    out = orc.layer(cfg, x, wr, wg, wu, wd, exact_logits=True)
    s = x @ wr.T
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    y = sum(p[:, e:e + 1] * _ffn(x, wg[e], wu[e], wd[e]) for e in range(E))
    np.testing.assert_allclose(out["y"], y, rtol=1e-10, atol=1e-12)


def test_gshard_einsum_dispatch_combine_with_drops(orc):
    """Tutorial, GShard pseudo-code: one-hot (S,E,C) dispatch mask filled in
    token order, einsum dispatch -> per-expert FFN on (E,C,M) -> einsum combine.
    Same y as the sparse oracle, including dropped assignments."""
    rng = np.random.default_rng(2)
    T, D, E, K, F = 40, 8, 4, 2, 8
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, E, F, E)
    wr[0] += 0.8  # skew the routing so capacity binds
    cfg = orc.Cfg(T=T, D=D, E=E, K=K, F=F, gating=orc.GATE_B, cap=1.0)
    out = orc.layer(cfg, x, wr, wg, wu, wd)
    C = out["capacity"]
    assert out["n_dropped"] > 0
    idx, w = out["idx"], out["w"]
    comb = np.zeros((T, E, C))
    fill = np.zeros(E, int)
    for t in range(T):
        for k in range(K):
            e = idx[t, k]
            if fill[e] < C:
                comb[t, e, fill[e]] = w[t, k]
            fill[e] += 1
    disp = (comb != 0).astype(np.float64)
    xin = np.einsum("sec,sm->ecm", disp, x)
    eo = np.stack([_ffn(xin[e], wg[e], wu[e], wd[e]) for e in range(E)])
    y = np.einsum("sec,ecm->sm", comb, eo)
    np.testing.assert_allclose(out["y"], y, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# P3 K=1 with renormalised gating: the router gets exactly zero gradient
# --------------------------------------------------------------------------
def test_k1_renormalised_router_gradient_is_exactly_zero(orc):
    rng = np.random.default_rng(3)
    T, D, E, F = 32, 16, 4, 24
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, E, F, E)
    cfg = orc.Cfg(T=T, D=D, E=E, K=1, F=F, gating=orc.GATE_B)
    out = orc.layer(cfg, x, wr, wg, wu, wd, dy=dy)
    assert np.all(out["w"] == 1.0)
    assert np.all(out["ds"] == 0.0) and np.all(out["dwr"] == 0.0) and np.all(out["drb"] == 0.0)
    cfgA = orc.Cfg(T=T, D=D, E=E, K=1, F=F, gating=orc.GATE_A)
    outA = orc.layer(cfgA, x, wr, wg, wu, wd, dy=dy)
    assert np.linalg.norm(outA["dwr"]) > 1e-3
    # with the aux loss switched on, the router gradient is the aux part alone
    outB = orc.layer(cfg, x, wr, wg, wu, wd, dy=dy, alpha=5e-4)
    dwr_aux = outB["dlogits_aux"].T @ x
    np.testing.assert_allclose(outB["dwr"], dwr_aux, rtol=1e-12, atol=1e-18)


def test_minimind_repro_norms(orc):
    """MiniMind issue section 3: the page's own 10-line repro, with torch used
    only as the page's random-number source; the gradient is the oracle's."""
    torch = pytest.importorskip("torch")
    g = gold("minimind_repro.json")
    B, H, E = g["B"], g["H"], g["E"]
    torch.manual_seed(g["seed"])
    x = torch.randn(B, H)
    gate_w = torch.randn(E, H)
    cases = [(1, orc.GATE_B), (2, orc.GATE_B), (1, orc.GATE_A)]
    ts = [torch.randn(B, k).double().numpy() for k, _ in cases]
    xn, wn = x.double().numpy(), gate_w.double().numpy()
    norms = []
    for (k, gating), t in zip(cases, ts):
        cfg = orc.Cfg(T=B, D=H, E=E, K=k, F=8, gating=gating)
        lg = orc.logits(cfg, xn, wn)
        idx, w, _, _ = orc.route(cfg, lg)
        ds = orc.gate_grad(cfg, lg, idx, w, t)
        norms.append(float(np.linalg.norm(ds.T @ xn)))
    assert norms[0] == 0.0                              # printed 1.249e-07 ~ 0
    assert abs(norms[1] - g["norm_k2_renorm_printed"]) < 0.005 * 12.23   # printed 1.223e+01
    # third printed value is unpinned; check against torch autograd instead
    xs = x.double()
    gw = gate_w.double().requires_grad_(True)
    sc = torch.softmax(xs @ gw.T, -1)
    wt, _ = torch.topk(sc, k=1, dim=-1)
    gr = torch.autograd.grad((wt * torch.from_numpy(ts[2])).sum(), gw)[0]
    assert abs(norms[2] - float(gr.norm())) < 1e-6 * float(gr.norm())


# --------------------------------------------------------------------------
# P7 sentinels: share additivity and the negative control
# --------------------------------------------------------------------------
def _share_case(orc, rng, **kw):
    T, D, E, K, F = 24, 8, 8, 3, 8
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, E, F, E)
    base = dict(T=T, D=D, E=E, K=K, F=F, **kw)
    return (x, wr, wg, wu, wd, dy), base


@pytest.mark.parametrize("score,gating,cap", [(0, 1, 0.0), (0, 0, 0.0), (0, 1, 1.0), (1, 1, 0.0)])
def test_sentinel_share_additivity(orc, score, gating, cap):
    rng = np.random.default_rng(4)
    (x, wr, wg, wu, wd, dy), base = _share_case(orc, rng, score=score, gating=gating, cap=cap)
    full = orc.layer(orc.Cfg(**base), x, wr, wg, wu, wd, dy=dy)
    parts = []
    for lo, hi in [(0, 5), (5, 8)]:
        sl = slice(lo, hi)
        parts.append(orc.layer(orc.Cfg(**base, lo=lo, hi=hi), x, wr, wg[sl], wu[sl], wd[sl], dy=dy))
    for key in ("y", "dx", "dwr", "drb", "ds"):
        np.testing.assert_allclose(parts[0][key] + parts[1][key], full[key], rtol=1e-11, atol=1e-13)
    for key in ("dwg", "dwu", "dwd"):
        np.testing.assert_allclose(np.concatenate([parts[0][key], parts[1][key]]), full[key],
                                   rtol=1e-12, atol=1e-14)
    # each share's counts are global, its rows are its own experts only
    assert parts[0]["counts_all"].tolist() == full["counts_all"].tolist()


def test_sentinel_bug_mode_signature(orc):
    """The page's signature: with the unmasked sentinel the loss and every
    expert-weight gradient are unchanged; only the router gradient moves."""
    sig = gold("sentinel_bug.json")
    assert sig["router_grad_norm_buggy"] > sig["router_grad_norm_reference"]
    rng = np.random.default_rng(5)
    (x, wr, wg, wu, wd, dy), base = _share_case(orc, rng)
    sl = slice(0, 4)
    ok = orc.layer(orc.Cfg(**base, lo=0, hi=4), x, wr, wg[sl], wu[sl], wd[sl], dy=dy)
    bad = orc.layer(orc.Cfg(**base, lo=0, hi=4, bug_mode=1), x, wr, wg[sl], wu[sl], wd[sl], dy=dy)
    np.testing.assert_array_equal(ok["y"], bad["y"])
    for key in ("dwg", "dwu", "dwd"):
        np.testing.assert_array_equal(ok[key], bad[key])
    assert np.linalg.norm(ok["dwr"] - bad["dwr"]) > 1e-3 * np.linalg.norm(ok["dwr"])
    # the masked sentinel slot carries dg = 0: a token routed only to remote
    # experts has ds = 0 under gating B
    remote = [t for t in range(base["T"]) if np.all(ok["idx"][t] >= 4)]
    for t in remote:
        assert np.all(ok["ds"][t] == 0.0)


# --------------------------------------------------------------------------
# P8 finite differences of the whole layer (fixed selection)
# --------------------------------------------------------------------------
def _fd_case(orc, score, gating, cap, n_shared=0, alpha=0.0, zlam=0.0, seed=6):
    rng = np.random.default_rng(seed)
    T, D, E, K, F = 6, 5, 5, 2, 4
    G = E + n_shared
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, E, F, G)
    rb = rng.standard_normal(E) * 0.1
    selb = rng.uniform(-0.1, 0.1, E).astype(np.float32) if score == 1 else None
    cfg = orc.Cfg(T=T, D=D, E=E, K=K, F=F, score=score, gating=gating, cap=cap, n_shared=n_shared)

    def loss(x, wr, rb, wg, wu, wd, idx0=None, cnt0=None):
        lg = orc.logits(cfg, x, wr, rb, exact=True)
        idx, w, _, _ = orc.route(cfg, lg, selb)
        if idx0 is not None:
            assert np.array_equal(idx, idx0), "selection moved under the perturbation"
        d = orc.dispatch(cfg, idx)
        y = orc.forward(cfg, x, wg, wu, wd, idx, w, d["slot_row"])
        L = float((dy * y).sum())
        if score == 0 and (alpha or zlam):
            losses, _ = orc.aux(cfg, lg, cnt0 if cnt0 is not None else d["counts_all"], alpha, zlam)
            L += losses[0] + losses[1]
        return L, lg, idx, w, d

    L0, lg, idx, w, d = loss(x, wr, rb, wg, wu, wd)
    # the selection margin must be far from the perturbation size
    key = lg if score == 0 else 1 / (1 + np.exp(-lg)) + (selb if selb is not None else 0)
    srt = np.sort(key, 1)[:, ::-1]
    assert np.min(srt[:, K - 1] - srt[:, K]) > 1e-4
    dlx = None
    if score == 0 and (alpha or zlam):
        _, dlx = orc.aux(cfg, lg, d["counts_all"], alpha, zlam)
    g = orc.backward(cfg, x, wr, wg, wu, wd, lg, idx, w, d["slot_row"], dy, dlx=dlx)
    # the router bias gradient is the column sum of ds
    params = dict(x=x, wr=wr, rb=rb, wg=wg, wu=wu, wd=wd)
    grads = dict(x=g["dx"], wr=g["dwr"], rb=g["drb"], wg=g["dwg"], wu=g["dwu"], wd=g["dwd"])
    h = 1e-6
    for name, P in params.items():
        flat = P.reshape(-1)
        fd = np.empty_like(flat)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + h
            Lp = loss(**params, idx0=idx, cnt0=d["counts_all"])[0]
            flat[i] = old - h
            Lm = loss(**params, idx0=idx, cnt0=d["counts_all"])[0]
            flat[i] = old
            fd[i] = (Lp - Lm) / (2 * h)
        an = grads[name].reshape(-1)
        err = np.max(np.abs(fd - an)) / max(np.max(np.abs(an)), 1e-3)
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("score,gating,cap,ns,alpha,zlam", [
    (0, 1, 0.0, 0, 0.0, 0.0), (0, 0, 0.0, 0, 0.0, 0.0), (0, 1, 0.0, 0, 0.05, 0.02),
    (0, 0, 1.0, 0, 0.0, 0.0), (1, 1, 0.0, 1, 0.0, 0.0), (1, 0, 0.0, 0, 0.0, 0.0)])
def test_finite_differences(orc, score, gating, cap, ns, alpha, zlam):
    _fd_case(orc, score, gating, cap, ns, alpha, zlam)


# --------------------------------------------------------------------------
# torch autograd on tiny fp64 inputs: an independent library check
# --------------------------------------------------------------------------
@pytest.mark.parametrize("score,gating", [(0, 0), (0, 1), (1, 1)])
def test_torch_autograd_tiny(orc, score, gating):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    T, D, E, K, F = 10, 6, 6, 3, 5
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, E, F, E)
    selb = rng.uniform(-0.1, 0.1, E).astype(np.float32) if score == 1 else None
    cfg = orc.Cfg(T=T, D=D, E=E, K=K, F=F, score=score, gating=gating)
    out = orc.layer(cfg, x, wr, wg, wu, wd, dy=dy, selb=selb, exact_logits=True)
    tx, twr = torch.tensor(x, requires_grad=True), torch.tensor(wr, requires_grad=True)
    twg, twu, twd = (torch.tensor(a, requires_grad=True) for a in (wg, wu, wd))
    s = tx @ twr.T
    idx = torch.from_numpy(out["idx"].astype(np.int64))
    if score == 0:
        p = torch.softmax(s, -1)
        sel = torch.gather(p, 1, idx)
        gw = sel if gating == 0 else sel / sel.sum(1, keepdim=True)
    else:
        sg = torch.sigmoid(torch.gather(s, 1, idx))
        gw = sg if gating == 0 else sg / sg.sum(1, keepdim=True)
    y = torch.zeros(T, D, dtype=torch.float64)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            a, b = tx[t] @ twg[e], tx[t] @ twu[e]
            y[t] = y[t] + gw[t, k] * ((torch.nn.functional.silu(a) * b) @ twd[e])
    L = (y * torch.from_numpy(dy)).sum()
    L.backward()
    np.testing.assert_allclose(out["y"], y.detach().numpy(), rtol=1e-10, atol=1e-12)
    for mine, ref in [("dx", tx), ("dwr", twr), ("dwg", twg), ("dwu", twu), ("dwd", twd)]:
        np.testing.assert_allclose(out[mine], ref.grad.numpy(), rtol=1e-9, atol=1e-12)


# --------------------------------------------------------------------------
# sampled / sparse-dy modes agree with the dense run
# --------------------------------------------------------------------------
def test_sparse_dy_and_column_subsets(orc):
    rng = np.random.default_rng(10)
    T, D, E, K, F = 30, 8, 6, 2, 12
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, E, F, E + 1)
    cfg = orc.Cfg(T=T, D=D, E=E, K=K, F=F, n_shared=1, cap=0.9)
    tok = np.array([3, 7, 8, 20, 29])
    dys = np.zeros_like(dy)
    dys[tok] = dy[tok]
    full = orc.layer(cfg, x, wr, wg, wu, wd, dy=dys)
    part = orc.backward(cfg, x, wr, wg, wu, wd, full["logits"], full["idx"], full["w"],
                        full["slot_row"], dy[tok], tok=tok, fsel=[1, 5, 11])
    np.testing.assert_allclose(part["dx"], full["dx"][tok], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(part["dwr"], full["dwr"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(part["dwg"], full["dwg"][:, :, [1, 5, 11]], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(part["dwd"], full["dwd"][:, [1, 5, 11], :], rtol=1e-13, atol=1e-15)
    ys = orc.forward(cfg, x, wg, wu, wd, full["idx"], full["w"], full["slot_row"], tok=tok)
    np.testing.assert_allclose(ys, full["y"][tok], rtol=1e-14)


def test_thread_count_does_not_change_results(orc):
    rng = np.random.default_rng(12)
    T, D, E, K, F = 40, 8, 6, 2, 8
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, E, F, E)
    cfg = orc.Cfg(T=T, D=D, E=E, K=K, F=F)
    n0 = orc.threads()
    try:
        orc.set_threads(1)
        a = orc.layer(cfg, x, wr, wg, wu, wd, dy=dy)
        orc.set_threads(5)
        b = orc.layer(cfg, x, wr, wg, wu, wd, dy=dy)
    finally:
        orc.set_threads(n0)
    for key in ("y", "dx", "dwr", "dwg", "dwd"):
        np.testing.assert_array_equal(a[key], b[key])


# ---------------------------------------------------------------------------
# sequence-wise balance loss and the load-driven bias update (next rows)
# ---------------------------------------------------------------------------
def test_seq_aux_worked_examples(orc):
    g = gold("seq_aux_example.json")["softmax"]
    p0 = np.array(g["p0"])
    lg = np.log(np.stack([p0, 1 - p0], 1))
    cfg = orc.Cfg(T=4, D=1, E=2, K=1, F=8)
    idx = np.array(g["choice"], np.int32)[:, None]
    L2, dl2 = orc.seq_aux(cfg, lg, idx, 2, g["alpha"])
    assert abs(L2 - g["S2"]["L"]) < 1e-12
    np.testing.assert_allclose(dl2[0], g["S2"]["dlogits_seq1"], atol=1e-15)
    np.testing.assert_allclose(dl2[1], g["S2"]["dlogits_seq1"], atol=1e-15)
    np.testing.assert_allclose(dl2[2:], 0.0, atol=1e-15)
    L4, _ = orc.seq_aux(cfg, lg, idx, 4, g["alpha"])
    assert abs(L4 - g["S4"]["L"]) < 1e-12
    with pytest.raises(ValueError):
        orc.seq_aux(cfg, lg, idx, 3, g["alpha"])


def test_seq_aux_sigmoid_worked_example(orc):
    g = gold("seq_aux_example.json")["sigmoid"]
    lg = np.array([[np.log(4.0), -np.log(4.0)], [np.log(1.5), -np.log(1.5)]])
    cfg = orc.Cfg(T=2, D=1, E=2, K=1, F=8, score=1)
    idx = np.array(g["choice"], np.int32)[:, None]
    L, dl = orc.seq_aux(cfg, lg, idx, g["S"], g["alpha"])
    assert abs(L - g["L"]) < 1e-12
    np.testing.assert_allclose(dl[0], g["dlogits_t0"], rtol=1e-12)


def test_seq_aux_full_sequence_is_batch_loss(orc):
    """S = T reduces to the batch balance loss (pinned by the worked example of
    section 8.5) on random routings, softmax scoring."""
    rng = np.random.default_rng(3)
    for E, K, T in [(4, 2, 32), (8, 1, 24), (6, 3, 12)]:
        cfg = orc.Cfg(T=T, D=1, E=E, K=K, F=8)
        lg = rng.normal(size=(T, E))
        idx, _, _, _ = orc.route(cfg, lg.astype(np.float32).astype(np.float64))
        counts = np.bincount(idx.ravel(), minlength=E)
        losses, dla = orc.aux(cfg, lg, counts, 0.02, 0.0)
        L, dls = orc.seq_aux(cfg, lg, idx, T, 0.02)
        assert abs(L - losses[0]) < 1e-14
        np.testing.assert_allclose(dls, dla, atol=1e-16)


@pytest.mark.parametrize("score", [0, 1])
def test_seq_aux_gradient_finite_differences(orc, score):
    """Central differences of the loss with the selection (and so f) held fixed."""
    rng = np.random.default_rng(11 + score)
    T, E, K, S = 12, 5, 2, 4
    cfg = orc.Cfg(T=T, D=1, E=E, K=K, F=8, score=score)
    lg = rng.normal(size=(T, E))
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    _, dl = orc.seq_aux(cfg, lg, idx, S, 0.05)
    h = 1e-6
    fd = np.zeros_like(lg)
    for t in range(T):
        for e in range(E):
            a = lg.copy(); a[t, e] += h
            b = lg.copy(); b[t, e] -= h
            fd[t, e] = (orc.seq_aux(cfg, a, idx, S, 0.05, False)[0]
                        - orc.seq_aux(cfg, b, idx, S, 0.05, False)[0]) / (2 * h)
    np.testing.assert_allclose(dl, fd, atol=1e-9 * np.abs(fd).max() + 1e-13, rtol=1e-6)


def test_bias_update_rule(orc):
    g = gold("seq_aux_example.json")["bias_update"]
    cfg = orc.Cfg(T=g["T"], D=1, E=g["E"], K=g["K"], F=8)
    b = orc.bias_update(cfg, g["counts"], g["gamma"], g["b_in"])
    b_in = np.array(g["b_in"], np.float32)
    gam = np.float32(g["gamma"])
    want = [b_in[e] + gam * np.float32(s) if s else b_in[e] for e, s in enumerate(g["expect_sign"])]
    np.testing.assert_array_equal(b, np.array(want, np.float32))
    # overloaded / underloaded is decided exactly in integers: a load one
    # above or below the mean moves the bias, the mean itself does not
    cfg2 = orc.Cfg(T=1000, D=1, E=3, K=1, F=8)
    b2 = orc.bias_update(cfg2, [334, 333, 333], 0.5, [0.0, 0.0, 0.0])
    np.testing.assert_array_equal(b2, np.array([-0.5, 0.5, 0.5], np.float32))


# ---------------------------------------------------------------------------
# noisy top-K selection and router-logit jitter (next row 2)
# ---------------------------------------------------------------------------
def test_noisy_topk_worked_example(orc):
    g = gold("noisy_topk_example.json")["noise"]
    s = np.array([g["s"]])
    eps, n = np.array([g["eps"]]), np.array([g["n"]])
    for K, gating in [(1, 0), (1, 1), (2, 1)]:
        cfg = orc.Cfg(T=1, D=1, E=4, K=K, F=8, gating=gating)
        idx, w, _, _, _ = orc.route_noisy(cfg, s, eps=eps, nlg=n)
        np.testing.assert_array_equal(idx[0], g[f"K{K}"]["idx"])
        if K == 1 and gating == 0:
            want = np.exp(1.9) / (np.exp(2.0) + np.exp(1.9) + 2.0)
            assert abs(w[0, 0] - want) < 1e-15
        elif K == 1:
            assert w[0, 0] == 1.0
        else:
            np.testing.assert_allclose(w[0], np.array([np.exp(1.9), np.exp(2.0)]) /
                                       (np.exp(1.9) + np.exp(2.0)), rtol=1e-15)
    cfg = orc.Cfg(T=1, D=1, E=4, K=1, F=8)
    assert orc.route(cfg, s)[0][0, 0] == g["without_noise_K1_idx"][0]


def test_jitter_worked_example(orc):
    g = gold("noisy_topk_example.json")["jitter"]
    s, u = np.array([g["s"]]), np.array([g["u"]])
    cfg = orc.Cfg(T=1, D=1, E=2, K=1, F=8, gating=0)
    idx, w, _, _, st = orc.route_noisy(cfg, s, jit=u, exact=True)
    assert idx[0, 0] == g["K1"]["idx"][0]
    np.testing.assert_allclose(st[0], g["s_jittered"], rtol=1e-15)
    assert abs(w[0, 0] - np.exp(1.01) / (np.exp(1.01) + np.exp(1.005))) < 1e-15
    assert orc.route(cfg, s)[0][0, 0] == g["without_jitter_K1_idx"][0]


def test_noise_and_jitter_reduce_to_plain_routing(orc):
    """eps = 0 and u = 1 give exactly the plain routing (special case)."""
    rng = np.random.default_rng(21)
    T, E, K = 40, 16, 4
    for gating in (0, 1):
        cfg = orc.Cfg(T=T, D=1, E=E, K=K, F=8, gating=gating)
        lg = rng.normal(size=(T, E)).astype(np.float32).astype(np.float64)
        a = orc.route(cfg, lg)
        b = orc.route_noisy(cfg, lg, jit=np.ones((T, E)), eps=np.zeros((T, E)),
                            nlg=rng.normal(size=(T, E)))
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_allclose(b[1], a[1], rtol=1e-14)
        np.testing.assert_allclose(b[2], a[2], rtol=1e-14)


def test_noise_only_selects(orc):
    """With noise the weights are the noise-free gate weights of the chosen
    set: gating B on s~ restricted to idx, summing to 1."""
    rng = np.random.default_rng(22)
    T, E, K = 50, 8, 3
    cfg = orc.Cfg(T=T, D=1, E=E, K=K, F=8, gating=1)
    lg = rng.normal(size=(T, E)).astype(np.float32).astype(np.float64)
    eps, n = rng.normal(size=(T, E)), rng.normal(size=(T, E))
    idx, w, _, probs, _ = orc.route_noisy(cfg, lg, eps=eps, nlg=n)
    sel = np.take_along_axis(probs, idx.astype(np.int64), 1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
    plain = orc.route(cfg, lg)[0]
    assert np.any(np.sort(idx, 1) != np.sort(plain, 1))  # the noise changed some choices


@pytest.mark.parametrize("gating", [0, 1])
def test_jitter_noise_torch_autograd_tiny(orc, gating):
    """Router gradients with jitter (and the noisy selection held fixed)
    against torch autograd of s~ = (x W_r^T) * u on tiny fp64 inputs."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(23)
    T, D, E, K, F = 10, 6, 6, 3, 5
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, E, F, E)
    cfg = orc.Cfg(T=T, D=D, E=E, K=K, F=F, gating=gating)
    u = rng.uniform(0.99, 1.01, size=(T, E)).astype(np.float32).astype(np.float64)
    eps = rng.normal(size=(T, E))
    lg = orc.logits(cfg, x, wr, exact=True)
    nlg = rng.normal(size=(T, E))
    idx, w, _, _, st = orc.route_noisy(cfg, lg, jit=u, eps=eps, nlg=nlg, exact=True)
    d = orc.dispatch(cfg, idx)
    y = orc.forward(cfg, x, wg, wu, wd, idx, w, d["slot_row"])
    bw = orc.backward(cfg, x, wr, wg, wu, wd, st, idx, w, d["slot_row"], dy,
                      jit=u.astype(np.float32))
    tx, twr = torch.tensor(x, requires_grad=True), torch.tensor(wr, requires_grad=True)
    s = (tx @ twr.T) * torch.tensor(u.astype(np.float32).astype(np.float64))
    tidx = torch.from_numpy(idx.astype(np.int64))
    p = torch.softmax(s, -1)
    sel = torch.gather(p, 1, tidx)
    gw = sel if gating == 0 else sel / sel.sum(1, keepdim=True)
    ty = torch.zeros(T, D, dtype=torch.float64)
    for t in range(T):
        for k in range(K):
            e = int(tidx[t, k])
            a, b = tx[t] @ torch.tensor(wg[e]), tx[t] @ torch.tensor(wu[e])
            ty[t] = ty[t] + gw[t, k] * ((torch.nn.functional.silu(a) * b) @ torch.tensor(wd[e]))
    (ty * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(bw["dwr"], twr.grad.numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(bw["dx"], tx.grad.numpy(), rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------------------
# expert-choice routing (next row 3)
# ---------------------------------------------------------------------------
def test_expert_choice_worked_example(orc):
    g = gold("expert_choice_example.json")
    cfg = orc.Cfg(T=g["T"], D=1, E=g["E"], K=g["K"], F=8, cap=g["c"])
    lg = np.log(np.array(g["p"]))
    r = orc.route_ec(cfg, lg)
    assert r["C"] == g["C"]
    np.testing.assert_array_equal(r["slot_row"], g["slot_row"])
    np.testing.assert_array_equal((r["slot_row"] >= 0).sum(1), g["times_taken"])
    np.testing.assert_allclose(r["w"], g["p"], rtol=1e-12)


def test_expert_choice_brute_force(orc):
    """Each local expert's taken set against Python sorted() on (-key, t)."""
    rng = np.random.default_rng(31)
    for T, E, K, cap, lo, hi in [(40, 6, 2, 1.0, 0, 6), (33, 5, 1, 1.3, 1, 4), (16, 4, 3, 0.0, 0, 4),
                                 (12, 8, 8, 2.0, 0, 8)]:
        cfg = orc.Cfg(T=T, D=1, E=E, K=K, F=8, lo=lo, hi=hi, cap=cap)
        lg = rng.normal(size=(T, E)).astype(np.float32).astype(np.float64)
        lg[3] = lg[5]  # exact ties between tokens
        r = orc.route_ec(cfg, lg)
        C = min(int(np.ceil((cap if cap > 0 else 1.0) * T * K / E)), T)
        assert r["C"] == C
        m = lg.max(1, keepdims=True)
        lse = (m + np.log(np.exp(lg - m).sum(1, keepdims=True)))[:, 0]
        key = (lg - lse[:, None]).astype(np.float32)
        row = 0
        for e in range(E):
            col = r["slot_row"][:, e]
            if not (lo <= e < hi):
                assert np.all(col == -2)
                continue
            want = sorted(range(T), key=lambda t: (-float(key[t, e]), t))[:C]
            got = np.nonzero(col >= 0)[0]
            np.testing.assert_array_equal(got, sorted(want))
            np.testing.assert_array_equal(col[got], np.arange(row, row + C))  # token order
            row += C
        np.testing.assert_array_equal(r["offsets"][: hi - lo + 1], np.arange(hi - lo + 1) * C)


def test_expert_choice_full_capacity_is_dense_soft_mixture(orc):
    """C = T: every expert takes every token, so the layer is the dense soft
    mixture y = sum_e softmax(s)_e FFN_e(x) -- the token-choice layer with
    K = E and truncated gating A."""
    rng = np.random.default_rng(32)
    T, D, E, F = 12, 6, 4, 5
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, E, F, E)
    cfg = orc.Cfg(T=T, D=D, E=E, K=E, F=F, cap=1.0)  # C = T
    lg = orc.logits(cfg, x, wr, exact=True)
    r = orc.route_ec(cfg, lg)
    assert r["C"] == T
    cw = r["cfg_w"]
    y_ec = orc.forward(cw, x, wg, wu, wd, r["idx"], r["w"], r["slot_row"])
    dense = orc.Cfg(T=T, D=D, E=E, K=E, F=F, gating=0)
    idx, w, _, _ = orc.route(dense, lg)
    d = orc.dispatch(dense, idx)
    y_tc = orc.forward(dense, x, wg, wu, wd, idx, w, d["slot_row"])
    np.testing.assert_allclose(y_ec, y_tc, rtol=1e-12, atol=1e-14)


def test_expert_choice_torch_autograd_tiny(orc):
    """Expert-choice forward and backward (selection held fixed) against torch
    autograd on tiny fp64 inputs, with local experts [1, 4) of 5."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(33)
    T, D, E, F = 14, 6, 5, 4
    x, wr, wg, wu, wd, dy = tiny_inputs(rng, T, D, E, F, 3)
    cfg = orc.Cfg(T=T, D=D, E=E, K=2, F=F, lo=1, hi=4)
    lg = orc.logits(cfg, x, wr, exact=True)
    r = orc.route_ec(cfg, lg)
    cw = r["cfg_w"]
    y = orc.forward(cw, x, wg, wu, wd, r["idx"], r["w"], r["slot_row"])
    bw = orc.backward(cw, x, wr, wg, wu, wd, lg, r["idx"], r["w"], r["slot_row"], dy)
    tx, twr = torch.tensor(x, requires_grad=True), torch.tensor(wr, requires_grad=True)
    twg, twu, twd = (torch.tensor(a, requires_grad=True) for a in (wg, wu, wd))
    p = torch.softmax(tx @ twr.T, -1)
    ty = torch.zeros(T, D, dtype=torch.float64)
    for t in range(T):
        for e in range(E):
            if r["slot_row"][t, e] < 0:
                continue
            g = e - 1
            a, b = tx[t] @ twg[g], tx[t] @ twu[g]
            ty[t] = ty[t] + p[t, e] * ((torch.nn.functional.silu(a) * b) @ twd[g])
    (ty * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-10, atol=1e-12)
    for mine, ref in [("dx", tx), ("dwr", twr), ("dwg", twg), ("dwu", twu), ("dwd", twd)]:
        np.testing.assert_allclose(bw[mine], ref.grad.numpy(), rtol=1e-9, atol=1e-12)
