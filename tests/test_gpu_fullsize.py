"""Parity at the full sizes of the five layer configurations, in the launch
configuration the benchmark times (same layer driver, device-generated
inputs).  The oracle cannot run the whole layer at these sizes, so:
  * routing (logits, top-K, counts, offsets, slot/row maps, drops) is compared
    for every token, bit-exactly -- the oracle computes all logits;
  * y, dx and the logit gradient are compared on sampled tokens (each depends
    only on its own token);
  * dW_r, d r_b and the expert-weight gradients come from a second backward
    with the upstream gradient zero outside the sampled tokens (no auxiliary
    loss term), which the oracle reproduces exactly from those tokens alone;
    expert-weight gradients are compared on sampled F-columns of every expert;
  * the sample is stratified: besides random tokens it holds the tokens of
    the first and last row of every 128-row m-tile (which includes every
    256-row tile edge) of the heaviest routed experts and of the shared
    expert, where ragged-tile and tile-boundary mistakes would show;
  * expert-weight gradients of the full (dense-dy) backward are compared on
    sampled F-columns of the heaviest, the lightest non-empty and any empty
    expert and of the shared expert, from every row of those groups.
"""
import numpy as np
import pytest

from mixture_experts_layer_23_amd import synthetic as S
from tests.gpu_common import TOL, as_f64, assert_close, assert_rows_close, note, ocfg, to_host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_23_amd import _lib
    _lib.lib()


# name: (workload, random tokens, sampled F-columns (None: all), heaviest
# routed experts whose m-tile edge rows join the token sample)
CASES = {
    "tiny_fp32": (S.WORKLOADS["tiny_fp32"], 256, None, 4),
    "minimind_k2_B": (S.WORKLOADS["minimind"], 48, 64, 4),
    "minimind_k1_B": (S.WORKLOADS["minimind"].with_(K=1), 48, 64, 4),
    "minimind_k2_A": (S.WORKLOADS["minimind"].with_(gating=S.GATE_A), 48, 64, 4),
    "minimind_k1_A": (S.WORKLOADS["minimind"].with_(K=1, gating=S.GATE_A), 48, 64, 4),
    "olmoe_share": (S.WORKLOADS["olmoe_share"], 24, 16, 4),
    "mixtral_cap": (S.WORKLOADS["mixtral_cap"], 12, 16, 2),
    "deepseek_v3": (S.WORKLOADS["deepseek_v3"], 16, 32, 8),
}

TILE_ROWS = 128


def edge_tokens(d, n_local, n_heavy, T, n_shared):
    """Tokens of the first and last row of every TILE_ROWS-row m-tile of the
    n_heavy largest routed groups and of the shared group."""
    offs = d["offsets"]
    sizes = np.diff(offs[: n_local + 1])
    heavy = np.argsort(-sizes, kind="stable")[:n_heavy]
    out = []
    for g in heavy:
        lo, hi = int(offs[g]), int(offs[g + 1])
        for r0 in range(lo, hi, TILE_ROWS):
            out += [d["row_token"][r0], d["row_token"][min(r0 + TILE_ROWS, hi) - 1]]
    if n_shared:
        for r0 in range(0, T, TILE_ROWS):
            out += [r0, min(r0 + TILE_ROWS, T) - 1]
    return np.array(out, np.int64), heavy


def host(t):
    return to_host(t)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(CASES))
def test_fullsize(name):
    from mixture_experts_layer_23_amd.layer import LayerSpec, MoELayer
    from oracle import oracle as O

    wl, n_rand, n_col, n_heavy = CASES[name]
    note(f"full-size {name}: {wl}")
    inp = S.device_inputs(wl)
    layer = MoELayer(LayerSpec.from_workload(wl), inp["wr"], inp["wg"], inp["wu"], inp["wd"],
                     inp["rb"], inp["selb"])
    layer.forward(inp["x"])
    layer.backward(inp["dy"])
    torch.cuda.synchronize()
    note("  gpu fwd+bwd done")
    x, wr, dy = host(inp["x"]), host(inp["wr"]), host(inp["dy"])
    rb = None if inp["rb"] is None else host(inp["rb"])
    selb = None if inp["selb"] is None else host(inp["selb"])
    wg, wu, wd = host(inp["wg"]), host(inp["wu"]), host(inp["wd"])
    oc = ocfg(wl)
    tol = TOL[wl.dtype]
    rng = np.random.default_rng(123)

    # routing, every token, bit-exact
    lg = O.logits(oc, x, wr, rb)
    g_lg = host(layer.logits)
    nbad = int(np.sum(g_lg != lg))
    note(f"  logits differing from the oracle: {nbad} of {lg.size}")
    assert_close("logits", g_lg, lg, 1e-5)
    idx, w, lse, probs = O.route(oc, lg, selb)
    np.testing.assert_array_equal(host(layer.topk_idx), idx)
    assert_close("topk_w", host(layer.topk_w), w, 1e-5)
    d = O.dispatch(oc, idx)
    np.testing.assert_array_equal(host(layer.counts), d["counts_all"])
    np.testing.assert_array_equal(host(layer.offsets), d["offsets"])
    np.testing.assert_array_equal(host(layer.slot_row), d["slot_row"])
    n = int(d["offsets"][-1])
    np.testing.assert_array_equal(host(layer.row_token)[:n], d["row_token"])
    assert int(host(layer.n_dropped)[0]) == d["n_dropped"]
    note(f"  routing bit-exact; rows {n}, dropped {d['n_dropped']}, loads "
         f"{d['counts_all'].tolist() if wl.E <= 16 else '...'}")

    # stratified token sample: random tokens + m-tile edge rows of the
    # heaviest experts and of the shared expert
    edges, heavy = edge_tokens(d, wl.n_local, n_heavy, wl.T, wl.n_shared)
    rand = rng.choice(wl.T, size=min(n_rand, wl.T), replace=False)
    tok = np.unique(np.concatenate([rand, edges])).astype(np.int32)
    note(f"  token sample: {len(tok)} tokens ({len(np.unique(edges))} tile-edge tokens of "
         f"experts {heavy.tolist()[:8]}{' and the shared expert' if wl.n_shared else ''})")

    # losses
    dl = None
    if wl.score == 0:
        losses, dl = O.aux(oc, lg, d["counts_all"], wl.alpha, wl.zlam)
        if layer.use_aux:
            gl = host(layer.losses)
            assert abs(gl[0] - losses[0]) <= 1e-5 * max(abs(losses[0]), 1e-30)
            assert abs(gl[1] - losses[1]) <= 1e-5 * max(abs(losses[1]), 1e-30)
            assert abs(gl[2] - losses[2]) <= 1e-5 * losses[2]
            note(f"  aux {gl[0]:.6e} z {gl[1]:.6e} z(raw) {gl[2]:.6e}")
    use_dl = dl if layer.use_aux else None

    # expert-weight gradients of the dense backward, copied before the
    # sparse backward below overwrites them: sampled F-columns of the
    # heaviest, the lightest non-empty and any empty routed expert, and of
    # the shared expert, from every row of those groups (oracle O10 on
    # columns)
    sizes = np.diff(d["offsets"][: wl.n_local + 1])
    wgroups = [int(heavy[0])] if wl.n_local else []
    nonempty = np.nonzero(sizes > 0)[0]
    if len(nonempty):
        wgroups.append(int(nonempty[np.argmin(sizes[nonempty])]))
    empty = np.nonzero(sizes == 0)[0]
    if len(empty):
        wgroups.append(int(empty[0]))
    if wl.n_shared:
        wgroups.append(wl.n_local)
    wgroups = sorted(set(wgroups))
    fcols = (np.arange(wl.F) if n_col is None
             else np.sort(rng.choice(wl.F, size=n_col, replace=False)))
    cs = torch.from_numpy(fcols.astype(np.int64)).cuda()
    dense_w = {g: (as_f64(host(layer.dw_gate[g][:, cs].contiguous())),
                   as_f64(host(layer.dw_up[g][:, cs].contiguous())),
                   as_f64(host(layer.dw_down[g][cs, :].contiguous()))) for g in wgroups}

    # sampled tokens: y, dx, ds (norm-wise over the sample and per token)
    tk = torch.from_numpy(tok.astype(np.int64)).cuda()
    y = O.forward(oc, x, wg, wu, wd, idx, w, d["slot_row"], tok=tok)
    gy = as_f64(host(layer.y[tk]))
    assert_close("y[sample]", gy, y, tol)
    assert_rows_close("y[sample]", gy, y, tol, zero_rows_exact=True)
    bw = O.backward(oc, x, wr, wg, wu, wd, lg, idx, w, d["slot_row"], as_f64(dy[tok]), tok=tok,
                    dlx=use_dl, want_wgrad=False, want_rgrad=False)
    gdx = as_f64(host(layer.dx[tk]))
    assert_close("dx[sample]", gdx, bw["dx"], tol)
    assert_rows_close("dx[sample]", gdx, bw["dx"], tol)
    assert_close("ds[sample]", host(layer.d_logits[tk]), bw["ds"], tol)
    note("  sampled y / dx / ds ok")

    dyf = as_f64(dy)
    for g in wgroups:
        ref = O.group_wgrad_cols(oc, x, wg, wu, wd, idx, w, d["slot_row"], dyf, g, fcols)
        rows_g = int(sizes[g]) if g < wl.n_local else wl.T
        for nm, got, r in zip(("dW_gate", "dW_up", "dW_down"), dense_w[g], ref):
            assert_close(f"{nm}[{g}] dense ({rows_g} rows)", got, r, tol)
    note(f"  dense-dy weight gradients ok on groups {wgroups}, {len(fcols)} columns")

    # weight gradients from a sparse upstream gradient: every expert, and
    # the router weight (which needs all tokens' logit gradients)
    dys = torch.zeros_like(inp["dy"])
    dys[tk] = inp["dy"][tk]
    layer.backward(dys, with_aux=False)
    torch.cuda.synchronize()
    fsel = None if n_col is None else np.sort(rng.choice(wl.F, size=min(n_col, 16), replace=False))
    bs = O.backward(oc, x, wr, wg, wu, wd, lg, idx, w, d["slot_row"], as_f64(dy[tok]), tok=tok,
                    fsel=fsel)
    assert_close("dW_r", host(layer.dw_r), bs["dwr"], tol)
    if rb is not None:
        assert_close("d_rbias", host(layer.d_rbias), bs["drb"], tol)
    if fsel is None:
        gw, uw, dw = layer.dw_gate, layer.dw_up, layer.dw_down
    else:
        cs = torch.from_numpy(fsel.astype(np.int64)).cuda()
        gw, uw, dw = layer.dw_gate[:, :, cs], layer.dw_up[:, :, cs], layer.dw_down[:, cs, :]
    assert_close("dW_gate", as_f64(host(gw.contiguous())), bs["dwg"], tol)
    assert_close("dW_up", as_f64(host(uw.contiguous())), bs["dwu"], tol)
    assert_close("dW_down", as_f64(host(dw.contiguous())), bs["dwd"], tol)
    if wl.K == 1 and wl.gating == S.GATE_B:
        assert np.all(host(layer.dw_r) == 0.0), "K=1 with gating B: router gradient must be 0"
    note("  weight gradients ok")
