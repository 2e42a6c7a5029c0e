"""Benchmark of the MoE layer (forward + backward) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--k K] [--gating A|B]

A step is one pass of the whole layer over one batch of synthetic tokens:
router GEMM, top-K gating, histogram/scan/permute, grouped SwiGLU expert
GEMMs, weighted combine, Switch/z losses and the full backward (expert dgrad
and wgrad, gating and router gradients).  Inputs and weights are resident in
HBM before the timed region.  Prints one JSON line.

The default workload is the MiniMind-like layer (T = 4096 tokens, D = 768,
E = 4 experts, top-2, SwiGLU F = 2048, bf16 with an fp32 router, gating B,
balance-loss coefficient 5e-4).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
F32_PEAK_TFLOPS = 157.3        # MI355X fp32 MFMA

GEMM_FLOPS_PER_ROW = {          # in units of D*F per row
    "gemm_gate_up_fwd": 4, "gemm_down_fwd": 2, "gemm_down_dgrad": 2, "gemm_down_wgrad": 2,
    "gemm_gate_up_dgrad": 4, "gemm_gate_up_wgrad": 4,
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="minimind")
    ap.add_argument("--k", type=int, default=None, help="override top-K")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override T (token sweeps of the routing / permute / combine kernels)")
    ap.add_argument("--gating", choices=["A", "B"], default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seq-len", type=int, default=0,
                    help="add the sequence-wise balance loss over sequences of this length")
    ap.add_argument("--seq-alpha", type=float, default=1e-3)
    ap.add_argument("--bias-gamma", type=float, default=0.0,
                    help="add the load-driven selection-bias step (sigmoid routing)")
    ap.add_argument("--jitter", action="store_true",
                    help="multiply the router logits by per-step U[0.99, 1.01] draws")
    ap.add_argument("--noise", action="store_true",
                    help="noisy top-K selection (noise router + per-step N(0,1) draws)")
    ap.add_argument("--routing", choices=["token", "expert"], default="token",
                    help="token choice (top-K per token) or expert choice (top-C tokens per "
                         "expert, softmax gating A)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed as one HIP graph (reported as ms_per_step_graph)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None)
    ap.add_argument("--no-isolated", action="store_true",
                    help="skip the untimed pass that times every kernel alone "
                         "(all kernels on one stream)")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (for HBM counter scaling)")
    return ap.parse_args()


def workload(args):
    from mixture_experts_layer_23_amd import synthetic as S
    wl = S.WORKLOADS[args.workload]
    if args.k is not None:
        wl = wl.with_(K=args.k)
    if args.tokens is not None:
        wl = wl.with_(T=args.tokens)
    if args.gating is not None:
        wl = wl.with_(gating=S.GATE_A if args.gating == "A" else S.GATE_B)
    if args.routing == "expert":
        wl = wl.with_(gating=S.GATE_A)  # a pair is weighted by its softmax probability
    return wl


def wl_name(wl):
    g = "A" if wl.gating == 0 else "B"
    sc = "softmax" if wl.score == 0 else "sigmoid"
    s = (f"{wl.name}: T={wl.T} D={wl.D} E={wl.E} K={wl.K} F={wl.F} {sc}/{g}"
         f" local=[{wl.lo},{wl.local_hi}) shared={wl.n_shared}")
    if wl.cap > 0:
        s += f" cap={wl.cap}"
    if wl.alpha:
        s += f" alpha={wl.alpha}"
    if wl.zlam:
        s += f" zloss={wl.zlam}"
    if wl.hot_bias:
        s += f" hot_bias={wl.hot_bias}"
    return s


def measured_traffic(kernel, wl):
    """HBM bytes per launch of `kernel` from the committed counter record
    (FETCH_SIZE and WRITE_SIZE runs scaled by a copy kernel of known size);
    None when there is no record for this kernel and workload or the GEMM
    source has changed since the counters were taken."""
    import glob
    import hashlib
    src = os.path.join(ROOT, "mixture_experts_layer_23_amd", "csrc", "gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for path in glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")):
        rec = json.load(open(path))
        if (rec.get("kernel") == kernel and rec.get("gemm_source_sha256") == sha
                and rec.get("workload_name") == wl_name(wl)):
            return rec["bytes_per_launch"]
    return None


def cpu_baseline(wl, host, n_tok, expert_choice=False):
    """The oracle as it stands, on a bounded sample of the same workload:
    routing of all T tokens (logits, top-K or expert choice, dispatch), then
    forward and the full backward (dx, dW_r and every expert-weight gradient
    contribution) of the first n_tok tokens.  Reported in tokens/s."""
    import numpy as np
    from oracle import oracle as O

    oc = O.Cfg(T=wl.T, D=wl.D, E=wl.E, K=wl.K, F=wl.F, lo=wl.lo, hi=wl.local_hi,
               n_shared=wl.n_shared, score=wl.score, gating=wl.gating, cap=wl.cap)
    x, wr, rb, selb, wg, wu, wd, dy = host
    tok = np.arange(n_tok, dtype=np.int32)
    t0 = time.perf_counter()
    lg = O.logits(oc, x, wr, rb)
    if expert_choice:
        r = O.route_ec(oc, lg)
        cw, idx, w, slot_row = r["cfg_w"], r["idx"], r["w"], r["slot_row"]
        counts = [r["C"]] * wl.E
    else:
        idx, w, lse, _ = O.route(oc, lg, selb)
        d = O.dispatch(oc, idx)
        cw, slot_row, counts = oc, d["slot_row"], d["counts_all"]
    O.forward(cw, x, wg, wu, wd, idx, w, slot_row, tok=tok)
    dl = None
    if wl.score == 0 and (wl.alpha or wl.zlam):
        _, dl = O.aux(oc, lg, counts, wl.alpha, wl.zlam)
    dyt = dy[tok].astype(np.float64) if dy.dtype != np.uint16 else \
        ((dy[tok].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    O.backward(cw, x, wr, wg, wu, wd, lg, idx, w, slot_row, dyt, tok=tok, dlx=dl)
    dt = time.perf_counter() - t0
    return dict(value=n_tok / dt, unit="tokens/s", cores=O.threads(), kind="oracle",
                sample=(f"routing of all {wl.T} tokens + forward and backward (dx, dW_r, all "
                        f"expert-weight gradient rows) of {n_tok} of them; {dt:.1f} s on "
                        f"{O.threads()} threads ({platform.processor() or platform.machine()})"))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(no multi-GPU path is implemented)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from mixture_experts_layer_23_amd import _lib as L
    from mixture_experts_layer_23_amd import synthetic as S
    from mixture_experts_layer_23_amd.layer import LayerSpec, MoELayer

    assert torch.cuda.is_available(), "needs a GPU"
    L.lib()
    if args.copy_calibration_mib:
        # one elementwise kernel that reads and writes exactly this many bytes:
        # the HBM counters of this launch calibrate FETCH_SIZE / WRITE_SIZE
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    wl = workload(args)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = S.device_inputs(wl, device="cuda")
    spec = LayerSpec.from_workload(wl, seq_len=args.seq_len,
                                   seq_alpha=args.seq_alpha if args.seq_len else 0.0,
                                   bias_gamma=args.bias_gamma,
                                   routing=(L.MOE_EXPERT_CHOICE if args.routing == "expert"
                                            else L.MOE_TOKEN_CHOICE))
    ec = spec.expert_choice
    u = eps = wn = None
    if args.jitter or args.noise:
        u, eps, wn = S.routing_noise(wl, device="cuda")
    layer = MoELayer(spec, inp["wr"], inp["wg"], inp["wu"], inp["wd"], inp["rb"],
                     None if ec else inp["selb"], w_noise=wn if args.noise else None)
    x, dy = inp["x"], inp["dy"]
    torch.cuda.synchronize()

    def step():
        layer.forward(x, jitter=u if args.jitter else None, noise_eps=eps if args.noise else None)
        layer.backward(dy)

    def timed(fn, live=None):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        if live:  # events around this kernel's launches, in the timed steps only
            L.timing_select(live)
            L.timing_enable(True)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1000.0 / max(args.steps, 1)

    # the kernel the roofline line is about: the largest total duration with
    # every kernel alone on the caller's stream (MOE_SERIAL_STREAMS, a short
    # untimed pass); beside other kernels on the side streams a duration also
    # counts the time the kernel shares the GPU
    os.environ["MOE_SERIAL_STREAMS"] = "1"
    try:
        for _ in range(max(args.warmup, 1)):
            step()
        torch.cuda.synchronize()
        L.timing_enable(True)
        for _ in range(max(min(args.steps, 5), 1)):
            step()
        torch.cuda.synchronize()
        L.timing_enable(False)
        dom = max(L.timing_report().items(), key=lambda kv: kv[1][1])[0]
    finally:
        del os.environ["MOE_SERIAL_STREAMS"]

    # untimed pass: per-kernel durations of every launch from HIP events the
    # library records on the stream each kernel runs on
    for _ in range(args.warmup):
        step()
    L.timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    L.timing_enable(False)
    kt = L.timing_report()

    # the timed region: kernel-by-kernel launches on the caller's stream (the
    # library overlaps independent backward parts on its side streams), with
    # events around the launches of the dominant kernel only, so its duration
    # is measured live in the same run
    ms = timed(step, live=dom)
    L.timing_enable(False)
    L.timing_select(None)
    kt_live = L.timing_report()
    ms_graph = None
    if args.graph:
        from mixture_experts_layer_23_amd.layer import StepGraph
        sg = StepGraph(layer, x, dy)
        ms_graph = timed(sg.replay)
        del sg

    # untimed pass with every kernel on the caller's stream (MOE_SERIAL_STREAMS):
    # each kernel's duration alone, next to the overlapped ones of the step
    kt_iso = None
    if not args.no_isolated:
        os.environ["MOE_SERIAL_STREAMS"] = "1"
        try:
            for _ in range(args.warmup):
                step()
            torch.cuda.synchronize()
            L.timing_enable(True)
            for _ in range(args.steps):
                step()
            torch.cuda.synchronize()
            L.timing_enable(False)
            kt_iso = L.timing_report()
        finally:
            del os.environ["MOE_SERIAL_STREAMS"]

    offsets = layer.offsets.cpu().numpy()
    counts = layer.counts.cpu().numpy()
    n_rows_local = int(offsets[wl.n_local]) if wl.n_local > 0 else 0
    rows = n_rows_local + wl.n_shared * wl.T
    n_dropped = None if ec else int(layer.n_dropped.cpu().numpy()[0])
    W = spec.width  # slots per token: K, or E under expert choice
    esz = 2 if wl.dtype == S.BF16 else 4
    kernels = {}
    gemm_flops = gemm_ms = 0.0
    for name, (n, tot) in kt.items():
        avg = tot / n
        e = dict(launches_per_step=n / max(args.steps, 1), avg_ms=avg)
        if name in GEMM_FLOPS_PER_ROW:
            fl = GEMM_FLOPS_PER_ROW[name] * wl.D * wl.F * rows
            e["tflops"] = fl / (avg * 1e-3) / 1e12
            gemm_flops += fl * n
            gemm_ms += tot
        kernels[name] = e
    # algorithmic bytes of the HBM-bound stages (per launch)
    Dsz = wl.D * esz
    stage_bytes = {
        "permute_gather": n_rows_local * Dsz * 2,
        "combine": rows * Dsz + wl.T * Dsz + wl.T * W * 8,
        "combine_bwd": n_rows_local * Dsz * 2 + wl.T * Dsz + wl.T * W * 8,
        "unpermute_dx": rows * Dsz + wl.T * Dsz + wl.T * W * 4,
        # logits read; p, keys of the local experts, sentinel columns written
        "ec_token": wl.T * wl.E * 4 * 2 + wl.T * wl.n_local * 4
                    + wl.T * (wl.E - wl.n_local) * 4,
        # keys read by three digit passes and the compaction; the local
        # columns of the slot table and two row maps written
        "ec_select": wl.T * wl.n_local * 4 * 4 + wl.T * wl.n_local * 4 + n_rows_local * 8,
        "route_select": wl.T * wl.E * 4 + wl.T * wl.K * 8 + wl.T * 4,
        "router_logits": wl.T * Dsz + wl.E * wl.D * 4 + wl.T * wl.E * 4,
        # x and W_r read; logits, top-K indices and weights, lse written
        "route_fused": wl.T * Dsz + wl.E * wl.D * 4 + wl.T * wl.E * 4 + wl.T * wl.K * 8
                       + wl.T * 4,
        # slot experts read (twice for the tiled rank); slot rows and the
        # two row maps written
        "permute_small": wl.T * wl.K * 8 + n_rows_local * 8,
        "permute_hist": wl.T * wl.K * 4,
        "permute_rank": wl.T * wl.K * 8 + n_rows_local * 8,
        "aux_single": wl.T * wl.E * 4 * (2 if wl.alpha or wl.zlam else 1),
        "router_wgrad": wl.T * Dsz + wl.T * wl.E * 4,
        "aux_partial": wl.T * wl.E * 4 * (2 if wl.alpha or wl.zlam else 1),
        # logits read twice (probabilities, then the gradient), routing read,
        # gradient written (read as well when accumulating)
        "seq_aux": wl.T * wl.E * 4 * (4 if layer.use_aux else 3) + wl.T * wl.K * 4,
    }
    for name, b in stage_bytes.items():
        if name in kernels:
            kernels[name]["gbs"] = b / (kernels[name]["avg_ms"] * 1e-3) / 1e9
            kernels[name]["hbm_frac"] = kernels[name]["gbs"] / HBM_PEAK_GBS
    kernels_iso = None
    gemm_iso = None
    if kt_iso:
        kernels_iso = {}
        fl_iso = ms_iso = 0.0
        for name, (n, tot) in kt_iso.items():
            avg = tot / n
            e = dict(avg_ms=avg)
            if name in GEMM_FLOPS_PER_ROW:
                fl = GEMM_FLOPS_PER_ROW[name] * wl.D * wl.F * rows
                e["tflops"] = fl / (avg * 1e-3) / 1e12
                e["frac_of_peak"] = e["tflops"] / (BF16_PEAK_TFLOPS if wl.dtype == S.BF16
                                                   else F32_PEAK_TFLOPS)
                fl_iso += fl * n
                ms_iso += tot
            if name in stage_bytes:
                e["gbs"] = stage_bytes[name] / (avg * 1e-3) / 1e9
                e["hbm_frac"] = e["gbs"] / HBM_PEAK_GBS
            kernels_iso[name] = e
        if ms_iso:
            t_iso = fl_iso / (ms_iso * 1e-3) / 1e12
            gemm_iso = {"tflops": t_iso,
                        "frac_of_peak": t_iso / (BF16_PEAK_TFLOPS if wl.dtype == S.BF16
                                                 else F32_PEAK_TFLOPS),
                        "ms_per_step": ms_iso / max(args.steps, 1)}
    n_live, tot_live = kt_live[dom]
    dom_avg = tot_live / n_live
    peak_t = BF16_PEAK_TFLOPS if wl.dtype == S.BF16 else F32_PEAK_TFLOPS
    if dom in GEMM_FLOPS_PER_ROW:
        ach = GEMM_FLOPS_PER_ROW[dom] * wl.D * wl.F * rows / (dom_avg * 1e-3) / 1e12
        roof = dict(kernel=dom, bound="mfma", achieved=ach, peak=peak_t, unit="TFLOP/s",
                    frac=ach / peak_t, traffic=measured_traffic(dom, wl),
                    per_launch=f"{GEMM_FLOPS_PER_ROW[dom]}*D*F flop x {rows} rows",
                    launches_timed=n_live)
    else:
        b = stage_bytes.get(dom, 0)
        ach = b / (dom_avg * 1e-3) / 1e9
        roof = dict(kernel=dom, bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=ach / HBM_PEAK_GBS, traffic=None, launches_timed=n_live)

    cpu = None
    if not args.no_cpu_baseline:
        host = (S.bf16_bits(inp["x"].float().cpu().numpy()) if wl.dtype == S.BF16
                else inp["x"].cpu().numpy(),
                inp["wr"].cpu().numpy(),
                None if inp["rb"] is None else inp["rb"].cpu().numpy(),
                None if inp["selb"] is None else inp["selb"].cpu().numpy(),
                *[t.cpu().view(torch.int16).numpy().view(np.uint16) if wl.dtype == S.BF16
                  else t.cpu().numpy() for t in (inp["wg"], inp["wu"], inp["wd"], inp["dy"])])
        n_tok = args.cpu_sample_tokens or min(wl.T, 4096)
        cpu = cpu_baseline(wl, host, n_tok, expert_choice=ec)

    out = {
        "metric": "MoE layer fwd+bwd tokens/s",
        "value": wl.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == S.BF16 else "f32",
        "data": "synthetic (seeded, on-device Philox normals)",
        "ms_per_step_graph": ms_graph,
        "config": {"workload": wl_name(wl), "launch": "eager",
                   "tokens": wl.T, "local_rows": n_rows_local,
                   "shared_rows": wl.n_shared * wl.T, "dropped": n_dropped,
                   "expert_load": counts.tolist() if wl.E <= 16 else None,
                   "seq_len": args.seq_len or None, "bias_gamma": args.bias_gamma or None,
                   "jitter": args.jitter or None, "noise": args.noise or None,
                   "routing": "expert choice" if ec else "token choice",
                   "expert_capacity": L.capacity(layer.cfg) if ec else None},
        "grouped_gemm": {"tflops": gemm_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None,
                         "frac_of_peak": (gemm_flops / (gemm_ms * 1e-3) / 1e12 / peak_t)
                         if gemm_ms else None,
                         "ms_per_step": gemm_ms / max(args.steps, 1)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        # the same kernels timed alone (untimed pass, one stream)
        "grouped_gemm_isolated": gemm_iso,
        "kernels_isolated": kernels_iso,
    }
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
