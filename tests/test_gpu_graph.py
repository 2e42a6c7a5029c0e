"""A forward + backward captured in a HIP graph gives, at every replay, the
same bits as the eager launches: replays separated by eager work of the
program (eager steps on the same layer, an unrelated torch kernel, host
synchronisation).  The layer's kernels are deterministic, so the comparison is
exact.  Covers the library's side-stream fork / join under capture and the
large-tile GEMM path (full-size MiniMind shape)."""
import pytest

torch = pytest.importorskip("torch")

from gpu_common import build_layer, note, to_dev  # noqa: E402
from mixture_experts_layer_23_amd import synthetic as S  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = {
    "minimind_full": S.WORKLOADS["minimind"],
    "olmoe_small": S.WORKLOADS["olmoe_share"].with_(T=300, D=128, E=16, K=4, F=128, hi=8),
    "mixtral_small": S.WORKLOADS["mixtral_cap"].with_(T=333, D=128, F=256),
    "deepseek_small": S.WORKLOADS["deepseek_v3"].with_(T=200, D=128, E=64, F=128),
}


def _outs(layer):
    return [t.clone() for t in (layer.y, layer.dx, layer.dw_r, layer.dw_gate, layer.dw_up,
                                layer.dw_down, layer.d_logits, layer.losses, layer.d_rbias)]


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replay_matches_eager(case):
    from mixture_experts_layer_23_amd.layer import LayerSpec, MoELayer, StepGraph
    wl = CASES[case]
    note(f"graph replay: {case} T={wl.T} D={wl.D} E={wl.E} K={wl.K} F={wl.F}")
    if wl.T >= 4096:
        inp = S.device_inputs(wl, device="cuda")
        layer = MoELayer(LayerSpec.from_workload(wl), inp["wr"], inp["wg"], inp["wu"], inp["wd"],
                         inp["rb"], inp["selb"])
        x, dy = inp["x"], inp["dy"]
    else:
        hin = S.host_inputs(wl, 0)
        layer = build_layer(wl, hin, torch)
        x, dy = to_dev(hin.x, torch), to_dev(hin.dy, torch)
    layer.forward(x)
    layer.backward(dy)
    torch.cuda.synchronize()
    ref = _outs(layer)
    g = StepGraph(layer, x, dy)
    for rep in range(4):
        # poison the outputs so that a replay which skipped a kernel shows
        for t in (layer.y, layer.dx, layer.dw_r, layer.dw_gate, layer.dw_up, layer.dw_down):
            t.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_outs(layer), ref)):
            assert torch.equal(a, b), f"{case}: replay {rep}, output {i} differs"
        # eager work of the program between replays
        a = torch.randn(256, 256, device="cuda")
        (a @ a).sum().item()
        layer.forward(x)
        layer.backward(dy)
        torch.cuda.synchronize()
