"""Benchmark of the dropless MoE layer hot path on one MI355X.

One step = one pass of the whole layer over one batch: route (fused x.W_r
projection + top-K), count/scan/permute, grouped SwiGLU MLP, combine.
Workload: the Mixtral-like layer, T=4096 tokens, H=4096, E=8 experts, top-2,
SwiGLU F=14336, bf16 activations/weights, fp32 router; synthetic seeded
inputs resident in HBM before the timed region.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu] [--no-mx]

Prints one JSON line: layer microseconds (the metric), per-stage times, the
grouped-GEMM TFLOP/s, route/permute/combine GB/s, the roofline of the dominant
launch pair (the two grouped GEMMs of moe_grouped_mlp, timed with events on the
stream they run on), and the CPU oracle timed on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-mx", action="store_true", help="skip the MXFP8 variant")
    ap.add_argument("--no-other", action="store_true", help="skip the other full-size workloads")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward kernels")
    ap.add_argument("--workload", choices=["dsv3_bf16", "sparse_share", "mixtral_mxfp8", "mixtral_mxfp4"],
                    default=None,
                    help="time only this other workload (its layer and grouped MLP) and print its line")
    ap.add_argument("--cpu-tokens", type=int, default=4096, help="tokens in the CPU oracle sample")
    return ap.parse_args()


def build(cfgname):
    import dropless_mixture_experts_radix_amd as D
    from workloads import get_config
    from workloads.gen import make_expert_weights, make_router_inputs, make_tokens

    cfg = get_config(cfgname)
    dt = {"bf16": D.BF16, "mxfp8": D.MXFP8, "mxfp4": D.MXFP4, "f32": D.F32}
    x = make_tokens(cfg).cuda()
    r = make_router_inputs(cfg)
    layer = D.MoELayer(cfg.T, cfg.H, cfg.E, cfg.K, cfg.F, dt[cfg.dtype], dt[cfg.x_dtype], L=cfg.local, e0=cfg.e0,
                       score=D.SIGMOID if cfg.score == "sigmoid" else D.SOFTMAX,
                       w_router=None if r["w_router"] is None else r["w_router"].cuda(),
                       bias=None if r["bias"] is None else r["bias"].cuda())
    for e in range(cfg.local):
        w1, w2 = make_expert_weights(cfg, cfg.e0 + e, device="cuda")
        layer.set_expert_weights(e, w1, w2)
        del w1, w2
    torch.cuda.synchronize()
    return cfg, layer, x, r


def time_steps(layer, x, steps, warmup):
    for _ in range(warmup):
        layer.forward(x)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(s)
    for _ in range(steps):
        layer.forward(x)
    t1.record(s)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_stages(layer, x, reps):
    """Per-stage times with events between the four calls (same stream)."""
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    acc = np.zeros(4)
    for _ in range(reps):
        ev[0].record(s)
        layer.route(x=x)
        ev[1].record(s)
        layer.permute(x)
        ev[2].record(s)
        layer.mlp()
        ev[3].record(s)
        layer.combine()
        ev[4].record(s)
        torch.cuda.synchronize()
        acc += [ev[i].elapsed_time(ev[i + 1]) for i in range(4)]
    return acc / reps * 1000.0  # us


def time_stages_graph(layer, x, reps):
    """Per-stage GPU times without host launch gaps: each stage captured
    `inner` times back to back in one HIP graph (same stream), the graph
    replayed `reps` times between two events."""
    stages = [(lambda: layer.route(x=x), 20), (lambda: layer.permute(x), 20), (layer.mlp, 2), (layer.combine, 20)]
    out = []
    for fn, inner in stages:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(inner):
                fn()
        torch.cuda.synchronize()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        out.append(t0.elapsed_time(t1) / (reps * inner) * 1000.0)
        del g
    return np.array(out)  # us


def time_graph(layer, x, reps):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        layer.forward(x)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / reps * 1000.0


def calibration_copy(nbytes=512 << 20):
    """One device-to-device copy of a known size (read nbytes, write nbytes).
    Under rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE give the factor that turns
    those counters into bytes for the kernels of the same run."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


GEMM_SOURCES = ["dropless_mixture_experts_radix_amd/csrc/gemm.hip", "dropless_mixture_experts_radix_amd/csrc/gemm_common.h"]
TRAFFIC_FILE = "profiles/mixtral_bf16_grouped_mlp_traffic.txt"


def gemm_source_sha():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per moe_grouped_mlp call (FETCH_SIZE + WRITE_SIZE, scaled by the
    calibration copy) from the committed counter summary, or None when the
    grouped GEMM sources changed since the counters were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), TRAFFIC_FILE)
    try:
        kv = {}
        with open(path) as fh:
            for ln in fh:
                if "=" in ln and not ln.lstrip().startswith("#"):
                    k, v = ln.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_sha256") != gemm_source_sha():
            return None
        return int(float(kv["hbm_bytes_per_call"]))
    except (OSError, KeyError, ValueError):
        return None


def algorithmic(cfg, N):
    T, H, E, K, F = cfg.T, cfg.H, cfg.E, cfg.K, cfg.F
    bx = 2
    route_b = T * H * bx + H * E * (4 if cfg.wr_dtype == "f32" else 2) + T * K * (2 + 4)
    row_b = H + H // 32 if cfg.dtype == "mxfp8" else H * bx
    permute_b = T * H * bx + N * row_b + T * K * 2 + T * K * 4 + N * 4
    combine_b = N * H * 2 + T * K * 4 + T * K * 4 + T * H * 2
    flops = 6.0 * N * H * F
    return route_b, permute_b, combine_b, flops


def cpu_baseline(cfg, layer, x, r, ntok):
    """The oracle as it stands, on the first `ntok` tokens of the same workload
    (route from the projection, count/permute, float64 grouped MLP, combine),
    scaled to the whole layer (x T/ntok).  Weights are converted to float64
    before the clock starts."""
    from oracle import moe_oracle as O
    from workloads.gen import make_expert_weights, to_numpy_f64
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    xs = to_numpy_f64(x[:ntok])
    wr = to_numpy_f64(r["w_router"])
    W1, W2 = [], []
    for e in range(cfg.local):
        w1, w2 = make_expert_weights(cfg, cfg.e0 + e, device="cuda")
        W1.append(to_numpy_f64(w1))
        W2.append(to_numpy_f64(w2))
        del w1, w2
    t0 = time.perf_counter()
    res = O.layer(xs, cfg.K, W1, W2, cfg.dtype, w_router=wr, score=cfg.score, e0=cfg.e0, L=cfg.local)
    dt = time.perf_counter() - t0
    del W1, W2
    # sanity: the sample's output agrees with the GPU layer on the same tokens
    gpu = to_numpy_f64(layer.out[:ntok])
    err = float(np.abs(gpu - res["out"]).max() / max(np.abs(res["out"]).max(), 1e-30))
    return {"value": dt * 1e6 * cfg.T / ntok, "unit": "us", "cores": int(cores), "kind": "oracle",
            "sample": f"first {ntok} of {cfg.T} tokens, whole layer (route, permute, fp64 grouped MLP, combine), "
                      f"{dt:.2f} s measured, scaled x{cfg.T // ntok}; max rel diff vs GPU on the sample {err:.2e}"}


def mx_variant(steps, warmup, name="mixtral_mxfp8"):
    cfg, layer, x, r = build(name)
    ms = time_steps(layer, x, steps, warmup)
    st = time_stages(layer, x, 10)
    N = int(layer.offsets[-1].item())
    route_b, permute_b, combine_b, flops = algorithmic(cfg, N)
    out = {"layer_us": ms * 1000.0, "stage_us": dict(zip(["route", "permute", "grouped_mlp", "combine"],
                                                         [round(v, 2) for v in st])),
           "grouped_gemm_tflops": flops / (st[2] * 1e-6) / 1e12,
           "peak_tflops": FP8_PEAK_TFLOPS if cfg.dtype == "mxfp8" else FP4_PEAK_TFLOPS,
           "grouped_gemm_frac_peak": flops / (st[2] * 1e-6) / 1e12 /
           (FP8_PEAK_TFLOPS if cfg.dtype == "mxfp8" else FP4_PEAK_TFLOPS),
           "permute_quantize_gbs": permute_b / (st[1] * 1e-6) / 1e9}
    del layer
    torch.cuda.empty_cache()
    return out


def graph_us(fn, inner=20, reps=5):
    """GPU time per call of fn: `inner` calls captured back to back in one HIP
    graph, replayed `reps` times between two events."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(inner):
            fn()
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / (reps * inner) * 1000.0
    del g
    return us


def other_workload(name, steps, warmup):
    """Layer time of another full-size workload of the method (not the metric's
    configuration): the DeepSeek-like layer (256 experts, Zipf-skewed loads,
    sigmoid scores) and the sparse large-top-K share (32 of 2304 experts, K=36,
    routed from given logits with masked tokens)."""
    cfg, layer, x, r = build(name)
    logits = None if r["logits"] is None else r["logits"].cuda()
    mask = None if r["mask"] is None else r["mask"].cuda()

    def fwd():
        layer.forward(x, logits=logits, mask=mask)

    for _ in range(warmup):
        fwd()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(s)
    for _ in range(steps):
        fwd()
    t1.record(s)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / steps * 1000.0
    N = int(layer.offsets[-1].item())
    flops = 6.0 * N * cfg.H * cfg.F
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(s)
    for _ in range(steps):
        layer.mlp()
    ev[1].record(s)
    torch.cuda.synchronize()
    mlp_us = ev[0].elapsed_time(ev[1]) / steps * 1000.0
    out = {"workload": f"{name}: T={cfg.T} H={cfg.H} E={cfg.E} local={cfg.local} K={cfg.K} F={cfg.F}",
           "layer_us": round(us, 2), "grouped_mlp_us": round(mlp_us, 2), "routed_rows": N,
           "grouped_gemm_tflops": round(flops / (mlp_us * 1e-6) / 1e12, 1)}
    if logits is None:
        import dropless_mixture_experts_radix_amd as D
        # route alone (projection + selection), and its group-limited variant
        # with a selection-only bias (8 groups of E/8 experts, 4 kept, gates x2.5)
        out["route_us"] = round(graph_us(lambda: layer.route(x=x)), 2)
        if cfg.E > 32 and cfg.E % 8 == 0 and cfg.K % 4 == 0:
            bias = layer.bias if layer.bias is not None else torch.zeros(cfg.E, device=x.device)
            out["grouped_route_us"] = round(graph_us(lambda: D.moe_route_topk_grouped(
                layer.ids, layer.probs, 8, 4, 2.5, x=x, w_prepared=layer.w_prep, w_dtype=layer.w_dtype, E=cfg.E,
                bias=bias, err=layer.err, workspace=layer.route_ws)), 2)
    del layer, x
    torch.cuda.empty_cache()
    return out


def backward_stages(layer, cfg, N):
    """GPU time per call (graph replays) of the routing backward on the layer's
    own maps: combine backward (d_y_perm and d_probs from a dout), permute
    backward (a token's gradient from its rows'), route backward (gate
    gradients with respect to the selected keys); algorithmic GB/s."""
    import dropless_mixture_experts_radix_amd as D
    T, H, K = cfg.T, cfg.H, cfg.K
    g = torch.Generator(device="cuda").manual_seed(99)
    dout = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    d_y = torch.empty_like(layer.y_perm)
    d_p = torch.empty((T, K), dtype=torch.float32, device="cuda")
    d_x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    d_z = torch.empty((T, K), dtype=torch.float32, device="cuda")
    t_cb = graph_us(lambda: D.moe_unpermute_combine_backward(dout, layer.y_perm, layer.slot_to_row, layer.probs,
                                                              d_y, d_p))
    t_pb = graph_us(lambda: D.moe_permute_backward(d_y, layer.slot_to_row, d_x))
    t_rb = graph_us(lambda: D.moe_route_backward(layer.ids, d_p, d_z, layer.score, probs=layer.probs, E=cfg.E))
    # data gradient of the grouped MLP (h recomputed, d_h, d_x): 3 GEMMs of 2 N H F flops each... GEMM1
    # recompute 4 N H F, d_a 2 N H F, d_x 4 N H F: 10 N H F
    F = cfg.F
    w1 = torch.empty((cfg.E, H, 2 * F), dtype=torch.bfloat16, device="cuda")
    w2 = torch.empty((cfg.E, F, H), dtype=torch.bfloat16, device="cuda")
    w1t = torch.empty(D.moe_prepared_weight_bytes(cfg.E, H, F, D.BF16, 5), dtype=torch.uint8, device="cuda")
    w2t = torch.empty(D.moe_prepared_weight_bytes(cfg.E, H, F, D.BF16, 6), dtype=torch.uint8, device="cuda")
    for e in range(cfg.E):  # the layer's own experts, regenerated from their seeds
        from workloads.gen import make_expert_weights
        a1, a2 = make_expert_weights(cfg, e, device="cuda")
        w1[e].copy_(a1)
        w2[e].copy_(a2)
    D.moe_prepare_weights_backward(w1, w2, w1t, w2t)
    # the MXFP8 panels: the forward's W1p and the backward's W1^T / W2^T, codes and scales
    mx = {k: torch.empty(D.moe_prepared_weight_bytes(cfg.E, H, F, D.MXFP8, k), dtype=torch.uint8, device="cuda")
          for k in (1, 2, 3, 4, 5, 6, 7, 8)}
    D.moe_prepare_weights(w1, w2, D.MXFP8, mx[1], mx[2], mx[3], mx[4])
    D.moe_prepare_weights_backward(w1, w2, mx[5], mx[6], mx[7], mx[8], dtype=D.MXFP8)
    del w1, w2, mx[2], mx[4]
    ws = torch.empty(D.moe_grouped_mlp_backward_workspace_bytes(layer.capacity, H, F, D.BF16), dtype=torch.uint8,
                     device="cuda")
    d_xp = torch.empty_like(layer.x_perm)
    bwd = lambda: D.moe_grouped_mlp_backward_data(layer.x_perm, layer.offsets, layer.w1p, w1t, w2t, d_y, d_xp, ws,
                                                  H, F)
    for _ in range(2):
        bwd()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        bwd()
    e1.record()
    torch.cuda.synchronize()
    t_mb = e0.elapsed_time(e1) / 3 * 1000.0
    # weight gradient (after the data gradient, from the h and d_h it left in ws): 6 N H F flops
    wws = torch.empty(D.moe_grouped_mlp_backward_weights_workspace_bytes(cfg.E, layer.capacity, H, F, D.BF16),
                      dtype=torch.uint8, device="cuda")
    dW1 = torch.empty((cfg.E, H, 2 * F), dtype=torch.float32, device="cuda")
    dW2 = torch.empty((cfg.E, F, H), dtype=torch.float32, device="cuda")
    wg = lambda: D.moe_grouped_mlp_backward_weights(layer.x_perm, layer.offsets, d_y, ws, dW1, dW2, wws, H, F)
    for _ in range(2):
        wg()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        wg()
    e1.record()
    torch.cuda.synchronize()
    t_wg = e0.elapsed_time(e1) / 3 * 1000.0
    # the same with MXFP8 operands (group-aware column-wise quantization included)
    del wws
    wws = torch.empty(D.moe_grouped_mlp_backward_weights_workspace_bytes(cfg.E, layer.capacity, H, F, D.MXFP8),
                      dtype=torch.uint8, device="cuda")
    wgm = lambda: D.moe_grouped_mlp_backward_weights(layer.x_perm, layer.offsets, d_y, ws, dW1, dW2, wws, H, F,
                                                     dtype=D.MXFP8)
    for _ in range(2):
        wgm()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        wgm()
    e1.record()
    torch.cuda.synchronize()
    t_wgm = e0.elapsed_time(e1) / 3 * 1000.0
    del ws, w1t, w2t, wws, dW1, dW2
    # the data gradient with MXFP8 operands (x_perm and d_y quantization included)
    ws = torch.empty(D.moe_grouped_mlp_backward_workspace_bytes(layer.capacity, H, F, D.MXFP8), dtype=torch.uint8,
                     device="cuda")
    bwdm = lambda: D.moe_grouped_mlp_backward_data(layer.x_perm, layer.offsets, mx[1], mx[5], mx[6], d_y, d_xp, ws,
                                                   H, F, dtype=D.MXFP8, w1p_scales=mx[3], w1t_scales=mx[7],
                                                   w2t_scales=mx[8])
    for _ in range(2):
        bwdm()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        bwdm()
    e1.record()
    torch.cuda.synchronize()
    t_mbm = e0.elapsed_time(e1) / 3 * 1000.0
    del ws, mx
    cb_bytes = T * H * 2 + 2 * N * H * 2 + T * K * 12
    pb_bytes = N * H * 2 + T * H * 2 + T * K * 4
    return {"combine_backward_us": round(t_cb, 2), "combine_backward_gbs": round(cb_bytes / (t_cb * 1e-6) / 1e9, 1),
            "permute_backward_us": round(t_pb, 2), "permute_backward_gbs": round(pb_bytes / (t_pb * 1e-6) / 1e9, 1),
            "route_backward_us": round(t_rb, 2),
            "grouped_mlp_backward_data_us": round(t_mb, 1),
            "grouped_mlp_backward_data_tflops": round(10.0 * N * H * F / (t_mb * 1e-6) / 1e12, 1),
            "grouped_mlp_backward_data_mxfp8_us": round(t_mbm, 1),
            "grouped_mlp_backward_data_mxfp8_tflops": round(10.0 * N * H * F / (t_mbm * 1e-6) / 1e12, 1),
            "grouped_mlp_backward_weights_us": round(t_wg, 1),
            "grouped_mlp_backward_weights_tflops": round(6.0 * N * H * F / (t_wg * 1e-6) / 1e12, 1),
            "grouped_mlp_backward_weights_mxfp8_us": round(t_wgm, 1),
            "grouped_mlp_backward_weights_mxfp8_tflops": round(6.0 * N * H * F / (t_wgm * 1e-6) / 1e12, 1),
            "note": "GPU time per call from HIP-graph replays (the MLP data gradient: events around 3 eager "
                    "calls; flops 10 N H F: h recomputed 4, d_a 2, d_x 4; the weight gradient likewise, 6 N H F, "
                    "its operand regrouping included); GB/s = algorithmic bytes (combine backward: dout, "
                    "y_perm read, d_y_perm written, maps/probs/d_probs; permute backward: rows read, token rows "
                    "written, map) / time"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported (the library has no multi-GPU "
              f"path)", file=sys.stderr)
        sys.exit(2)
    if a.workload:
        line = other_workload(a.workload, a.steps, a.warmup)
        line.update({"metric": "MoE layer us (" + a.workload + ")", "value": line["layer_us"], "unit": "us",
                     "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "higher_is_better": False,
                     "dtype": "bf16", "data": "synthetic"})
        print(json.dumps(line), flush=True)
        return
    calibration_copy()
    cfg, layer, x, r = build("mixtral_bf16")
    layer.forward(x)
    torch.cuda.synchronize()
    N = int(layer.offsets[-1].item())
    torch.cuda.synchronize()
    ms = time_steps(layer, x, a.steps, a.warmup)
    st_eager = time_stages(layer, x, 20)
    st = time_stages_graph(layer, x, 5)
    gus = time_graph(layer, x, a.steps)
    route_b, permute_b, combine_b, flops = algorithmic(cfg, N)
    t_route, t_perm, t_comb = st[0], st[1], st[3]
    t_mlp = st_eager[2]  # events on the launch stream around the call
    tflops = flops / (t_mlp * 1e-6) / 1e12
    line = {
        "metric": "MoE layer us; grouped-GEMM TFLOPS + permute/combine GB/s, 1 MI355X",
        "value": round(ms * 1000.0, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mixtral_bf16: T=4096 H=4096 E=8 K=2 SwiGLU F=14336, bf16 rows/weights, "
                               "fp32 router", "tokens": cfg.T, "routed_rows": N},
        "stage_us": {"route": round(t_route, 2), "permute": round(t_perm, 2), "grouped_mlp": round(t_mlp, 2),
                     "combine": round(t_comb, 2)},
        "stage_us_note": "route/permute/combine: GPU time per call from HIP-graph replays of 20 back-to-back "
                         "calls; grouped_mlp: events around the eager call",
        "stage_us_eager": {k: round(float(v), 2) for k, v in
                           zip(["route", "permute", "grouped_mlp", "combine"], st_eager)},
        "graph_replay_us": round(gus, 2),
        "grouped_gemm_tflops": round(tflops, 1),
        "route_gbs": round(route_b / (t_route * 1e-6) / 1e9, 1),
        "permute_gbs": round(permute_b / (t_perm * 1e-6) / 1e9, 1),
        "combine_gbs": round(combine_b / (t_comb * 1e-6) / 1e9, 1),
        "roofline": {"kernel": "moe_grouped_mlp: k_gemm_bf16<1> (GEMM1+SwiGLU) + k_gemm_bf16<0> (GEMM2) "
                               "+ k_splitk_reduce<1,0>",
                     "bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(),
                     "traffic_unit": "HBM bytes per launch", "algorithmic_flops_per_launch": flops},
    }
    if not a.no_backward:
        try:
            line["backward"] = backward_stages(layer, cfg, N)
        except Exception as ex:  # report, do not hide the main line
            line["backward"] = {"error": repr(ex)}
    if not a.no_mx:
        try:
            del layer
            torch.cuda.empty_cache()
            for name, key in (("mixtral_mxfp8", "mxfp8"), ("mixtral_mxfp4", "mxfp4")):
                try:
                    line[key] = mx_variant(max(a.steps // 2, 5), a.warmup, name)
                except Exception as ex:  # report, do not hide the main line
                    line[key] = {"error": repr(ex)}
            cfg, layer, x, r = build("mixtral_bf16")
            layer.forward(x)
            torch.cuda.synchronize()
        except Exception as ex:  # report, do not hide the main line
            line["mx"] = {"error": repr(ex)}
    if not a.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg, layer, x, r, a.cpu_tokens)
    if not a.no_other:
        del layer, x
        torch.cuda.empty_cache()
        line["other_workloads"] = []
        for name in ("dsv3_bf16", "sparse_share"):
            try:
                line["other_workloads"].append(other_workload(name, 10, 3))
            except Exception as ex:  # report, do not hide the main line
                line["other_workloads"].append({"workload": name, "error": repr(ex)})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
