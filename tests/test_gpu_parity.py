"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Integer routing results are compared bit-exactly;
floating-point results with the norm-wise relative error of gpu_common
(1e-5 fp32 layers, 2e-2 bf16 layers with fp32 accumulation)."""
import numpy as np
import pytest

from mixture_experts_layer_23_amd import synthetic as S
from tests.gpu_common import (TOL, as_f64, assert_close, assert_rows_close, build_layer, note,
                              ocfg, rel_err, to_dev, to_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_23_amd import _lib
    _lib.lib()  # must load; no fallback


def O():
    from oracle import oracle
    return oracle


# ---------------------------------------------------------------------------
# routing on given logits: bit-exact indices
# ---------------------------------------------------------------------------
ROUTE_CASES = [
    (257, 4, 1, 0, 0, False), (257, 4, 2, 0, 1, True), (300, 8, 2, 0, 1, False),
    (129, 64, 8, 0, 1, True), (100, 64, 8, 0, 0, False), (70, 256, 8, 1, 1, False),
    (70, 256, 8, 1, 0, True), (33, 3, 3, 0, 1, True), (65, 1000, 16, 0, 1, False),
    (40, 16, 16, 1, 1, False), (1, 5, 2, 0, 1, False)]


@pytest.mark.parametrize("T,E,K,score,gating,ties", ROUTE_CASES)
def test_route_given_logits_bit_exact(T, E, K, score, gating, ties):
    from mixture_experts_layer_23_amd import _lib as L
    note(f"route T={T} E={E} K={K} score={score} gating={gating} ties={ties}")
    lg = S.random_logits(T, E, seed=T * 7 + E, scale=2.0, ties=ties)
    selb = None
    if score == 1:
        selb = np.random.default_rng(E).uniform(-0.1, 0.1, E).astype(np.float32)
    oc = O().Cfg(T=T, D=64, E=E, K=K, F=64, score=score, gating=gating)
    idx, w, lse, _ = O().route(oc, lg, selb)
    cfg = L.make_config(T, 64, E, K, 64, score_fn=score, gating=gating, dtype=L.MOE_F32)
    d_lg = to_dev(lg, torch)
    d_idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    d_w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    d_lse = torch.empty(T, dtype=torch.float32, device="cuda")
    L.moe_route(cfg, None, None, None, to_dev(selb, torch), d_lg, d_idx, d_w, d_lse,
                L.MOE_ROUTE_LOGITS_GIVEN)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(d_idx), idx)
    assert_close("topk_w", to_host(d_w), w, 1e-5)
    assert_close("lse", to_host(d_lse), lse, 1e-5)


# router logits from x on the fp64 matrix cores (E > 16): 32 x 64 tiles with
# 4, 2 or 1 k-groups per workgroup (fewer than 512, 512..1023, 1024+ tiles),
# ragged tokens and experts, fewer k-slabs than k-groups (D = 64)
ROUTER_TILED = [(200, 128, 64, S.BF16), (1000, 64, 100, S.F32), (16384, 128, 64, S.BF16),
                (16000, 192, 100, S.BF16), (32768, 64, 64, S.F32)]


# the few-expert router (E <= 16, logits and top-K in one kernel): W_r read
# through the caches (<= 32 KB) or staged in LDS (waves then loop over several
# token pairs), partial 4-vector chunks of D, a single token
ROUTER_SKINNY = [(777, 768, 4, S.BF16), (4097, 2048, 16, S.BF16), (1000, 1088, 8, S.F32),
                 (1, 64, 3, S.F32), (16384, 512, 16, S.BF16), (3001, 4096, 8, S.BF16)]


@pytest.mark.parametrize("T,D,E,dt", ROUTER_TILED + ROUTER_SKINNY)
def test_router_logits_tiled(T, D, E, dt):
    from mixture_experts_layer_23_amd import _lib as L
    note(f"router logits T={T} D={D} E={E} dtype={dt}")
    rng = np.random.default_rng(T + 3 * D + 7 * E)
    xf = rng.standard_normal((T, D)).astype(np.float32)
    x = S.bf16_bits(xf) if dt == S.BF16 else xf
    wr = (rng.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)
    rb = rng.uniform(-0.5, 0.5, E).astype(np.float32)
    K = min(4, E)
    oc = O().Cfg(T=T, D=D, E=E, K=K, F=64)
    lg = O().logits(oc, x, wr, rb)
    idx, w, _, _ = O().route(oc, lg)
    cfg = L.make_config(T, D, E, K, 64, dtype=L.MOE_BF16 if dt == S.BF16 else L.MOE_F32)
    d_lg = torch.empty(T, E, dtype=torch.float32, device="cuda")
    d_idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    d_w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    L.moe_route(cfg, to_dev(x, torch), to_dev(wr, torch), to_dev(rb, torch), None, d_lg, d_idx,
                d_w, None)
    torch.cuda.synchronize()
    g = to_host(d_lg)
    # one rounding of an fp64 sum: equal to the oracle's unless the sum falls
    # within fp64 rounding of a binary32 rounding boundary
    nbad = int(np.sum(g != lg))
    note(f"  logits differing: {nbad} of {g.size}")
    assert nbad <= 2
    assert_close("logits", g, lg, 1e-6)
    # rows whose logits all agree: the top-K indices are bit-exact
    same = np.all(g == lg, axis=1)
    gi = to_host(d_idx)
    np.testing.assert_array_equal(gi[same], idx[same])
    # a row with a differing logit: the GPU's indices are a valid top-K of its
    # own logits (descending keys, lower index first among equal keys)
    for t in np.nonzero(~same)[0]:
        assert_valid_topk(g[t], gi[t])
    assert_close("topk_w", to_host(d_w), w, 1e-5)


def assert_valid_topk(keys, picked):
    """picked lists distinct experts in descending key order, equal keys by
    ascending index, and no unpicked expert beats the last pick."""
    keys = np.asarray(keys, np.float32)
    picked = [int(e) for e in picked]
    assert len(set(picked)) == len(picked)
    for a, b in zip(picked, picked[1:]):
        assert keys[a] > keys[b] or (keys[a] == keys[b] and a < b)
    last = picked[-1]
    for e in range(len(keys)):
        if e not in picked:
            assert keys[e] < keys[last] or (keys[e] == keys[last] and e > last)


def test_sigmoid_key_bit_exact_on_a_sweep():
    """sig32 on the GPU equals the oracle's bit for bit: each row holds two
    adjacent binary32 logits, so the top-1 on sig32(s) depends on the last bit
    of the rounded sigmoid (equal keys -> index 0, else index 1)."""
    from mixture_experts_layer_23_amd import _lib as L
    T, E = 8192, 2
    s0 = np.linspace(-30, 30, T, dtype=np.float32)
    s1 = np.nextafter(s0, np.float32(np.inf)).astype(np.float32)
    lg = np.stack([s0, s1], 1)
    b = np.zeros(E, np.float32)
    oc = O().Cfg(T=T, D=64, E=E, K=1, F=64, score=1, gating=1)
    idx, _, _, _ = O().route(oc, lg, b)
    assert 0 < int(idx.sum()) < T  # both outcomes occur
    cfg = L.make_config(T, 64, E, 1, 64, score_fn=1, gating=1, dtype=L.MOE_F32)
    d_idx = torch.empty(T, 1, dtype=torch.int32, device="cuda")
    d_w = torch.empty(T, 1, dtype=torch.float32, device="cuda")
    L.moe_route(cfg, None, None, None, to_dev(b, torch), to_dev(lg, torch), d_idx, d_w, None,
                L.MOE_ROUTE_LOGITS_GIVEN)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(d_idx), idx)


# ---------------------------------------------------------------------------
# permutation: bit-exact integer maps and gather
# ---------------------------------------------------------------------------
PERM_CASES = [
    (257, 4, 2, 0, 4, 0.0, 0), (1000, 8, 2, 0, 8, 1.25, 0), (513, 64, 8, 0, 32, 0.0, 0),
    (300, 16, 4, 4, 12, 1.0, 1), (77, 256, 8, 0, 256, 0.0, 1), (256, 4, 2, 0, 4, 1.1, 0),
    (1, 4, 2, 0, 4, 0.0, 0), (50, 6, 3, 6, 6, 0.0, 1), (64, 5, 5, 0, 5, 0.3, 0),
    # one-workgroup path with 16 and 32 rounds of slots in registers
    (3000, 8, 4, 0, 8, 0.0, 0), (7000, 16, 4, 4, 16, 1.2, 1),
    # beyond the one-workgroup path (32768 slots, 256 experts): the tiled
    # histogram / scan / rank kernels
    (4500, 64, 8, 8, 40, 1.0, 1), (40, 300, 4, 0, 300, 0.0, 1), (4097, 512, 8, 0, 512, 1.5, 0)]


@pytest.mark.parametrize("T,E,K,lo,hi,cap,ns", PERM_CASES)
def test_permute_bit_exact(T, E, K, lo, hi, cap, ns):
    from mixture_experts_layer_23_amd import _lib as L
    note(f"permute T={T} E={E} K={K} lo={lo} hi={hi} cap={cap} ns={ns}")
    rng = np.random.default_rng(T + 31 * E)
    # skewed routing so capacity binds on the first experts
    p = np.exp(-np.arange(E) / max(E / 3, 1.0))
    idx = np.array([rng.choice(E, size=K, replace=False, p=p / p.sum()) for _ in range(T)],
                   np.int32)
    D = 128
    x = S.bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    oc = O().Cfg(T=T, D=D, E=E, K=K, F=64, lo=lo, hi=hi, cap=cap, n_shared=ns)
    want = O().dispatch(oc, idx)
    cfg = L.make_config(T, D, E, K, 64, lo, hi, ns, dtype=L.MOE_BF16, capacity_factor=cap)
    rows = L.rows_max(cfg)
    G = hi - lo + ns
    i32 = dict(dtype=torch.int32, device="cuda")
    counts = torch.empty(E, **i32)
    offsets = torch.empty(G + 1, **i32)
    slot_row = torch.empty(T * K, **i32)
    row_token = torch.full((rows,), -7, **i32)
    row_slot = torch.full((rows,), -7, **i32)
    nd = torch.empty(4, **i32)
    xp = torch.zeros(rows, D, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(L.workspace_size(cfg), dtype=torch.uint8, device="cuda")
    L.moe_permute(cfg, to_dev(idx, torch), to_dev(x, torch), counts, offsets, slot_row, row_token,
                  row_slot, nd, xp, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(counts), want["counts_all"])
    np.testing.assert_array_equal(to_host(offsets), want["offsets"])
    np.testing.assert_array_equal(to_host(slot_row), want["slot_row"])
    n = int(want["offsets"][-1])
    np.testing.assert_array_equal(to_host(row_token)[:n], want["row_token"])
    np.testing.assert_array_equal(to_host(row_slot)[:n], want["row_slot"])
    assert int(to_host(nd)[0]) == want["n_dropped"]
    nr = int(want["offsets"][hi - lo])
    np.testing.assert_array_equal(to_host(xp)[:nr], x[want["row_token"][:nr]])


# ---------------------------------------------------------------------------
# the whole layer, forward + backward, at sizes the oracle checks densely
# ---------------------------------------------------------------------------
SMALL = {
    "tiny_fp32": S.WORKLOADS["tiny_fp32"],
    "minimind_k2_B": S.WORKLOADS["minimind"].with_(T=512, D=256, F=512),
    "minimind_k2_A": S.WORKLOADS["minimind"].with_(T=512, D=256, F=512, gating=S.GATE_A),
    "minimind_k1_A": S.WORKLOADS["minimind"].with_(T=384, D=256, F=512, K=1, gating=S.GATE_A),
    "olmoe_share": S.WORKLOADS["olmoe_share"].with_(T=300, D=128, E=16, K=4, F=128, hi=8),
    "olmoe_share_A": S.WORKLOADS["olmoe_share"].with_(T=200, D=128, E=16, K=4, F=128, hi=8,
                                                      gating=S.GATE_A),
    "mixtral_cap": S.WORKLOADS["mixtral_cap"].with_(T=333, D=128, F=256),
    "deepseek_v3": S.WORKLOADS["deepseek_v3"].with_(T=200, D=128, E=64, F=128),
    "fp32_sentinel_cap": S.WORKLOADS["tiny_fp32"].with_(T=190, E=6, K=3, hi=4, cap=0.8,
                                                        n_shared=1),
}


def run_layer(wl, seed=0):
    hin = S.host_inputs(wl, seed)
    layer = build_layer(wl, hin, torch)
    x, dy = to_dev(hin.x, torch), to_dev(hin.dy, torch)
    layer.forward(x)
    layer.backward(dy)
    torch.cuda.synchronize()
    return hin, layer


def oracle_layer(wl, hin):
    o = O()
    oc = ocfg(wl)
    lg = o.logits(oc, hin.x, hin.wr, hin.rb)
    idx, w, lse, probs = o.route(oc, lg, hin.selb)
    d = o.dispatch(oc, idx)
    y = o.forward(oc, hin.x, hin.wg, hin.wu, hin.wd, idx, w, d["slot_row"])
    aux = wl.score == 0 and (wl.alpha or wl.zlam)
    losses = dl = None
    if wl.score == 0:
        losses, dl = o.aux(oc, lg, d["counts_all"], wl.alpha, wl.zlam)
    bw = o.backward(oc, hin.x, hin.wr, hin.wg, hin.wu, hin.wd, lg, idx, w, d["slot_row"],
                    as_f64(hin.dy), dlx=dl if aux else None)
    return dict(logits=lg, idx=idx, w=w, lse=lse, y=y, losses=losses, dl=dl, **d, **bw)


def compare_layer(wl, hin, layer, ref, check_acts=True):
    tol = TOL[wl.dtype]
    g = lambda t: to_host(t)
    lg = g(layer.logits)[: wl.T]
    nbad = int(np.sum(lg != ref["logits"]))
    note(f"  logits differing from the oracle: {nbad} of {lg.size}")
    assert_close("logits", lg, ref["logits"], 1e-5)
    np.testing.assert_array_equal(g(layer.topk_idx), ref["idx"])
    assert_close("topk_w", g(layer.topk_w), ref["w"], 1e-5)
    np.testing.assert_array_equal(g(layer.counts), ref["counts_all"])
    np.testing.assert_array_equal(g(layer.offsets), ref["offsets"])
    np.testing.assert_array_equal(g(layer.slot_row), ref["slot_row"])
    n = int(ref["offsets"][-1])
    np.testing.assert_array_equal(g(layer.row_token)[:n], ref["row_token"])
    assert int(g(layer.n_dropped)[0]) == ref["n_dropped"]
    if check_acts and n > 0:
        o = O()
        grp = np.searchsorted(ref["offsets"], np.arange(n), side="right") - 1
        a, b, h, oo = o.expert_rows(ocfg(wl), hin.x, hin.wg, hin.wu, hin.wd, grp,
                                    ref["row_token"])
        act = as_f64(g(layer.act)[:n])
        errs = [assert_close("act_a", act[:, : wl.F], a, tol),
                assert_close("act_b", act[:, wl.F:], b, tol),
                assert_close("h", as_f64(g(layer.h)[:n]), h, tol),
                assert_close("o_perm", as_f64(g(layer.o_perm)[:n]), oo, tol)]
        note(f"  act/h/o errs {['%.2e' % e for e in errs]}")
    errs = {}
    errs["y"] = assert_close("y", as_f64(g(layer.y)[: wl.T]), ref["y"], tol)
    errs["dx"] = assert_close("dx", as_f64(g(layer.dx)[: wl.T]), ref["dx"], tol)
    errs["y_row"] = assert_rows_close("y", as_f64(g(layer.y)[: wl.T]), ref["y"], tol,
                                      zero_rows_exact=True)
    errs["dx_row"] = assert_rows_close("dx", as_f64(g(layer.dx)[: wl.T]), ref["dx"], tol)
    errs["ds"] = assert_close("d_logits", g(layer.d_logits)[: wl.T], ref["ds"], tol)
    errs["dwr"] = assert_close("dW_r", g(layer.dw_r), ref["dwr"], tol)
    if hin.rb is not None:
        errs["drb"] = assert_close("d_rbias", g(layer.d_rbias), ref["drb"], tol)
    errs["dwg"] = assert_close("dW_gate", as_f64(g(layer.dw_gate)), ref["dwg"], tol)
    errs["dwu"] = assert_close("dW_up", as_f64(g(layer.dw_up)), ref["dwu"], tol)
    errs["dwd"] = assert_close("dW_down", as_f64(g(layer.dw_down)), ref["dwd"], tol)
    if ref["losses"] is not None and layer.use_aux:
        l = g(layer.losses)
        assert abs(l[0] - ref["losses"][0]) <= 1e-5 * max(abs(ref["losses"][0]), 1e-30)
        assert abs(l[2] - ref["losses"][2]) <= 1e-5 * max(abs(ref["losses"][2]), 1e-30)
    note("  errs " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    return errs


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_parity(name):
    wl = SMALL[name]
    note(f"layer {name}: {wl}")
    hin, layer = run_layer(wl)
    ref = oracle_layer(wl, hin)
    compare_layer(wl, hin, layer, ref)


# Router backward for more than 16 experts: the fp32 matrix-core GEMMs (E a
# multiple of 4) with ragged token, model-dimension, expert and split edges,
# and the SIMT fallback (E not a multiple of 4); both dtypes, router bias on.
ROUTER_BWD = {
    "mfma_fp32_E132_T1000_D192": S.WORKLOADS["tiny_fp32"].with_(
        T=1000, D=192, E=132, K=4, F=64, hot_bias=0.5, alpha=1e-3),
    "mfma_bf16_E36_T777_D320": S.WORKLOADS["minimind"].with_(
        T=777, D=320, E=36, K=3, F=128, hot_bias=1.0),
    "mfma_bf16_sigmoid_E260_T513": S.WORKLOADS["deepseek_v3"].with_(
        T=513, D=128, E=260, K=6, F=64, hot_bias=0.3),
    "simt_fp32_E18": S.WORKLOADS["tiny_fp32"].with_(T=300, D=128, E=18, K=2, F=64,
                                                    hot_bias=0.5),
    "simt_bf16_E30": S.WORKLOADS["minimind"].with_(T=450, D=192, E=30, K=4, F=64, hot_bias=1.0),
}


@pytest.mark.parametrize("name", list(ROUTER_BWD))
def test_router_backward_many_experts(name):
    wl = ROUTER_BWD[name]
    note(f"router backward {name}: {wl}")
    hin, layer = run_layer(wl)
    ref = oracle_layer(wl, hin)
    compare_layer(wl, hin, layer, ref, check_acts=False)


def test_k1_renormalised_router_gradient_is_exactly_zero():
    wl = S.WORKLOADS["minimind"].with_(T=512, D=256, F=512, K=1, gating=S.GATE_B, alpha=0.0)
    hin, layer = run_layer(wl)
    assert np.all(to_host(layer.topk_w) == 1.0)
    assert np.all(to_host(layer.d_logits) == 0.0)
    assert np.all(to_host(layer.dw_r) == 0.0)
    # with the balance loss on, the router gradient is the aux part alone
    wl2 = wl.with_(alpha=5e-4)
    hin2, layer2 = run_layer(wl2)
    ref = oracle_layer(wl2, hin2)
    assert_close("dW_r aux only", to_host(layer2.dw_r), ref["dwr"], TOL[wl.dtype])
    dwr_aux = ref["dl"].T @ as_f64(hin2.x)
    assert_close("dW_r == aux part", to_host(layer2.dw_r), dwr_aux, TOL[wl.dtype])


def test_sentinel_slots_carry_no_router_gradient_and_shares_add_up():
    base = S.WORKLOADS["olmoe_share"].with_(T=256, D=128, E=16, K=2, F=128)
    full = base.with_(lo=0, hi=16)
    hin, lf = run_layer(full)
    parts = []
    for lo, hi in [(0, 8), (8, 16)]:
        wl = base.with_(lo=lo, hi=hi)
        hs = S.host_inputs(wl)
        hs.wg, hs.wu, hs.wd = hin.wg[lo:hi], hin.wu[lo:hi], hin.wd[lo:hi]
        layer = build_layer(wl, hs, torch)
        layer.forward(to_dev(hin.x, torch))
        layer.backward(to_dev(hin.dy, torch))
        torch.cuda.synchronize()
        parts.append(layer)
        # a token routed only to remote experts has ds == 0 exactly (gating B)
        idx = to_host(layer.topk_idx)
        remote = np.all((idx < lo) | (idx >= hi), axis=1)
        assert np.all(to_host(layer.d_logits)[remote] == 0.0)
    tol = TOL[base.dtype]
    for name in ("y", "dx"):
        s = sum(as_f64(to_host(getattr(p, name))) for p in parts)
        assert_close(f"{name} shares", s, as_f64(to_host(getattr(lf, name))), 2 * tol)
    s = sum(to_host(p.dw_r).astype(np.float64) for p in parts)
    assert_close("dW_r shares", s, to_host(lf.dw_r), 2 * tol)


EDGE = {
    "T1": S.WORKLOADS["minimind"].with_(T=1, D=128, F=128),
    "ragged_T": S.WORKLOADS["minimind"].with_(T=131, D=128, F=128, E=8, K=3),
    "K_equals_E": S.WORKLOADS["tiny_fp32"].with_(T=70, E=4, K=4, gating=S.GATE_B),
    "all_sentinel_with_shared": S.WORKLOADS["deepseek_v3"].with_(T=64, D=128, E=8, K=2, F=128,
                                                                 lo=3, hi=3),
    "all_sentinel": S.WORKLOADS["olmoe_share"].with_(T=64, D=128, E=8, K=2, F=128, lo=8, hi=8),
    "tiny_capacity": S.WORKLOADS["mixtral_cap"].with_(T=100, D=128, F=128, cap=0.05),
    "single_expert_K1": S.WORKLOADS["minimind"].with_(T=100, D=64, F=64, E=1, K=1),
    "minimal_dims_sigmoid_A_shared": S.WORKLOADS["deepseek_v3"].with_(
        T=50, D=64, F=64, E=16, K=4, gating=S.GATE_A),
    "capacity_exactly_even": S.WORKLOADS["mixtral_cap"].with_(T=257, D=128, F=128, cap=1.0),
    "K_equals_E_64": S.WORKLOADS["tiny_fp32"].with_(T=40, D=64, F=64, E=64, K=64),
    # more than 8 slots per token: the generic slot loops of the combine, its
    # backward, the gating backward and the un-permute
    "K12_softmax_B": S.WORKLOADS["tiny_fp32"].with_(T=150, E=24, K=12, F=64),
    "K10_sigmoid_A": S.WORKLOADS["deepseek_v3"].with_(T=120, D=128, E=32, K=10, F=64,
                                                      gating=S.GATE_A),
    # long batches: the un-permute takes 4 (K <= 2) or 2 (K <= 4) tokens per
    # wave; ragged last wave
    "unpermute_4_per_wave": S.WORKLOADS["minimind"].with_(T=16387, D=128, F=64, E=8, K=2),
    "unpermute_2_per_wave": S.WORKLOADS["tiny_fp32"].with_(T=8195, D=192, F=64, E=6, K=3),
    "many_empty_experts": S.WORKLOADS["deepseek_v3"].with_(T=9, D=128, E=256, K=8, F=128),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases(name):
    wl = EDGE[name]
    note(f"edge {name}: {wl}")
    hin, layer = run_layer(wl)
    ref = oracle_layer(wl, hin)
    compare_layer(wl, hin, layer, ref, check_acts=False)


def test_all_tokens_to_one_expert_via_given_logits():
    from mixture_experts_layer_23_amd.layer import LayerSpec, MoELayer
    wl = S.WORKLOADS["minimind"].with_(T=200, D=128, F=128, E=4, K=1, gating=S.GATE_A)
    hin = S.host_inputs(wl)
    layer = build_layer(wl, hin, torch)
    lg = np.zeros((wl.T, wl.E), np.float32)
    lg[:, 2] = 5.0
    layer.logits[: wl.T].copy_(torch.from_numpy(lg))
    layer.forward(to_dev(hin.x, torch), logits_given=True)
    torch.cuda.synchronize()
    assert to_host(layer.counts).tolist() == [0, 0, 200, 0]
    off = to_host(layer.offsets)
    assert off.tolist() == [0, 0, 0, 200, 200]
    o = O()
    oc = ocfg(wl)
    idx, w, _, _ = o.route(oc, lg)
    d = o.dispatch(oc, idx)
    y = o.forward(oc, hin.x, hin.wg, hin.wu, hin.wd, idx, w, d["slot_row"])
    assert_close("y", as_f64(to_host(layer.y)), y, TOL[wl.dtype])


def test_serial_streams_give_identical_results(monkeypatch):
    """The backward's side-stream overlap changes no result: with
    MOE_SERIAL_STREAMS every kernel runs on the caller's stream, and all
    outputs equal the overlapped run's bit for bit."""
    wl = SMALL["deepseek_v3"]
    _, a = run_layer(wl)
    snap = {k: to_host(getattr(a, k)).copy() for k in
            ("y", "dx", "dw_r", "dw_gate", "dw_up", "dw_down", "d_logits")}
    monkeypatch.setenv("MOE_SERIAL_STREAMS", "1")
    _, b = run_layer(wl)
    for k, v in snap.items():
        np.testing.assert_array_equal(to_host(getattr(b, k)), v, err_msg=k)


def test_deterministic_across_runs():
    wl = SMALL["olmoe_share"]
    _, a = run_layer(wl)
    snap = {k: to_host(getattr(a, k)).copy() for k in
            ("y", "dx", "dw_r", "dw_gate", "dw_up", "dw_down", "d_logits", "slot_row")}
    _, b = run_layer(wl)
    for k, v in snap.items():
        np.testing.assert_array_equal(to_host(getattr(b, k)), v, err_msg=k)
