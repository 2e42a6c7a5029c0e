"""One expert group whose row operands exceed 2 GiB.

The grouped GEMMs read row operands through buffer descriptors with 32-bit
offsets; the descriptors are based at the tile's first row (row-major
operands) or the k-slab's first row (k-major operands), so a group of any
size is read in full.  Here a single expert takes all T = 40000 tokens with
F = 32768: the saved activations a|b and their gradients are 40000 x 65536
bf16 (5.2 GB) and h is 2.6 GB, so rows past 2^31 bytes are a large share of
every operand that the down-projection forward, the gate/up data gradient
and both weight gradients read.  Checked against the oracle on sampled tokens
(including the last rows) and on sampled F-columns of the dense-dy weight
gradients from all 40000 rows, for the default kernel selection and with the
256-row, 256 x 256 and persistent kernels forced.
"""
import numpy as np
import pytest

from mixture_experts_layer_23_amd import synthetic as S
from tests.gpu_common import (TOL, as_f64, assert_close, assert_rows_close, build_layer, note,
                              ocfg, to_dev, to_host)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

WL = S.WORKLOADS["minimind"].with_(T=40000, D=256, E=1, K=1, F=32768, alpha=0.0,
                                   gating=S.GATE_A)


@pytest.fixture(scope="module", autouse=True)
def gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_cache = {}


def reference():
    if "ref" not in _cache:
        from oracle import oracle as O
        hin = S.host_inputs(WL)
        oc = ocfg(WL)
        lg = O.logits(oc, hin.x, hin.wr, hin.rb)
        idx, w, _, _ = O.route(oc, lg)
        d = O.dispatch(oc, idx)
        assert int(d["offsets"][-1]) == WL.T  # one group holding every token
        rng = np.random.default_rng(5)
        # tokens on both sides of 2^31 bytes of h (row 32768) and of a|b
        # (row 16384), the last rows, and random ones
        tok = np.unique(np.concatenate([
            rng.choice(WL.T, 24, replace=False), [0, 16383, 16384, 32767, 32768, WL.T - 1],
            np.arange(WL.T - 8, WL.T)])).astype(np.int32)
        y = O.forward(oc, hin.x, hin.wg, hin.wu, hin.wd, idx, w, d["slot_row"], tok=tok)
        bw = O.backward(oc, hin.x, hin.wr, hin.wg, hin.wu, hin.wd, lg, idx, w, d["slot_row"],
                        as_f64(hin.dy[tok]), tok=tok, want_wgrad=False, want_rgrad=False)
        fcols = np.sort(rng.choice(WL.F, 12, replace=False))
        wref = O.group_wgrad_cols(oc, hin.x, hin.wg, hin.wu, hin.wd, idx, w, d["slot_row"],
                                  as_f64(hin.dy), 0, fcols)
        _cache["ref"] = (hin, tok, y, bw, fcols, wref)
    return _cache["ref"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("gemm_cfg", [None, "2", "5", "7"])
def test_group_over_2gib(gemm_cfg, monkeypatch):
    hin, tok, y, bw, fcols, wref = reference()
    if gemm_cfg is not None:
        monkeypatch.setenv("MOE_GEMM_CFG", gemm_cfg)
    note(f"one group of {WL.T} rows, F = {WL.F}: a|b {WL.T * 2 * WL.F * 2 / 1e9:.1f} GB, "
         f"h {WL.T * WL.F * 2 / 1e9:.1f} GB; MOE_GEMM_CFG={gemm_cfg}")
    layer = build_layer(WL, hin, torch)
    layer.forward(to_dev(hin.x, torch))
    layer.backward(to_dev(hin.dy, torch))
    torch.cuda.synchronize()
    tol = TOL[WL.dtype]
    tk = torch.from_numpy(tok.astype(np.int64)).cuda()
    gy = as_f64(to_host(layer.y[tk]))
    gdx = as_f64(to_host(layer.dx[tk]))
    assert_close("y", gy, y, tol)
    assert_rows_close("y", gy, y, tol, zero_rows_exact=True)
    assert_close("dx", gdx, bw["dx"], tol)
    assert_rows_close("dx", gdx, bw["dx"], tol)
    cs = torch.from_numpy(fcols.astype(np.int64)).cuda()
    got = (as_f64(to_host(layer.dw_gate[0][:, cs].contiguous())),
           as_f64(to_host(layer.dw_up[0][:, cs].contiguous())),
           as_f64(to_host(layer.dw_down[0][cs, :].contiguous())))
    for nm, g, r in zip(("dW_gate", "dW_up", "dW_down"), got, wref):
        assert_close(nm, g, r, tol)
    note("  y, dx and weight-gradient columns ok")
    del layer
    torch.cuda.empty_cache()
