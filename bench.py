"""Benchmark of the dropless MoE layer hot path on one MI355X.

One step = one pass of the whole layer over one batch: route (fused x.W_r
projection + top-K), count/scan/permute, grouped SwiGLU MLP, combine.
Workload: the Mixtral-like layer, T=4096 tokens, H=4096, E=8 experts, top-2,
SwiGLU F=14336, bf16 activations/weights, fp32 router; synthetic seeded
inputs resident in HBM before the timed region.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--iters 160] [--no-cpu] [--no-mx]

Prints one JSON line: layer microseconds (the metric: the mean of the K timed
steps), the layer and every stage over 160 single calls timed with events both
cold (a 512 MiB buffer written just before each call, outside the events:
more than the 256 MB last-level cache and the L2s) and warm (HIP-graph
replays of back-to-back calls), as median, p10 and p90; the grouped-GEMM
TFLOP/s and the route/permute/combine GB/s, each as a fraction of the
datasheet peak and of the ceilings measured in the same run by the library's
calibration kernels (streaming copy, read and write; matrix-core loops); the
roofline of the dominant launch (moe_grouped_mlp, timed with events on the
stream it runs on); and the CPU oracle timed on bounded samples.
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
FLUSH_BYTES = 512 << 20


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
    ap.add_argument("--iters", type=int, default=160, help="single calls timed per stage, cold and warm")
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


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def _one_thread():
    """Context that limits the BLAS pool to one thread (numpy's own loops are
    single-threaded anyway)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except Exception:
        import contextlib
        return contextlib.nullcontext()


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, layer, x, r, ntok):
    """The oracle as it stands, stage by stage, on the first `ntok` tokens of
    the same workload: route (projection + top-K), count/permute and combine
    on one thread; the float64 grouped MLP on all BLAS threads of the process
    affinity mask.  Scaled to the whole layer (x T/ntok).  Weights are
    converted to float64 before the clock starts."""
    from oracle import moe_oracle as O
    from workloads.gen import make_expert_weights, to_numpy_f64
    cores = _blas_threads()
    xs = to_numpy_f64(x[:ntok])
    wr = to_numpy_f64(r["w_router"])
    W1, W2 = [], []
    for e in range(cfg.local):
        w1, w2 = make_expert_weights(cfg, cfg.e0 + e, device="cuda")
        W1.append(to_numpy_f64(w1))
        W2.append(to_numpy_f64(w2))
        del w1, w2
    t = {}
    with _one_thread():
        t0 = time.perf_counter()
        logits = O.router_logits(xs, wr)
        ids, probs = O.route_topk(logits, cfg.K, cfg.score)
        t["route"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        perm = O.count_and_permute(ids, cfg.e0, cfg.local, xs, E_global=cfg.E)
        t["permute"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    y, _ = O.grouped_mlp(perm["x_perm"], perm["offsets"], W1, W2, cfg.dtype)
    t["grouped_mlp"] = time.perf_counter() - t0
    with _one_thread():
        t0 = time.perf_counter()
        out = O.combine(y, perm["slot_to_row"], probs, "bf16")
        t["combine"] = time.perf_counter() - t0
    del W1, W2
    dt = sum(t.values())
    # sanity: the sample's output agrees with the GPU layer on the same tokens
    gpu = to_numpy_f64(layer.out[:ntok])
    err = float(np.abs(gpu - out).max() / max(np.abs(out).max(), 1e-30))
    scale = cfg.T / ntok
    return {"value": round(dt * 1e6 * scale, 1), "unit": "us", "cores": int(cores), "kind": "oracle",
            "stage_us": {k: round(v * 1e6 * scale, 1) for k, v in t.items()},
            "cpu": _cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"first {ntok} of {cfg.T} tokens, whole layer: route, count/permute and combine on 1 thread, "
                      f"fp64 grouped MLP on {cores} BLAS threads; {dt:.2f} s measured, scaled x{scale:g}; max rel "
                      f"diff vs GPU on the sample {err:.2e}"}


def cpu_one_core(name, ntok):
    """The whole oracle layer on one thread for another workload, on its
    first `ntok` tokens (all of them when ntok >= T), scaled to T tokens;
    min of 3 runs."""
    from oracle import moe_oracle as O
    from workloads import get_config
    from workloads.gen import make_expert_weights, make_router_inputs, make_tokens, to_numpy_f64
    cfg = get_config(name)
    ntok = min(ntok, cfg.T)
    x = to_numpy_f64(make_tokens(cfg)[:ntok])
    r = make_router_inputs(cfg)
    W1, W2 = [], []
    for e in range(cfg.local):
        w1, w2 = make_expert_weights(cfg, cfg.e0 + e, device="cpu")
        W1.append(to_numpy_f64(w1))
        W2.append(to_numpy_f64(w2))
    kw = dict(score=cfg.score, e0=cfg.e0, L=cfg.local)
    if r["logits"] is not None:
        kw["logits"] = to_numpy_f64(r["logits"][:ntok])
    else:
        kw["w_router"] = to_numpy_f64(r["w_router"])
    if r["mask"] is not None:
        kw["mask"] = r["mask"][:ntok].numpy().astype(bool)
    best = None
    with _one_thread():
        for _ in range(3):
            t0 = time.perf_counter()
            O.layer(x, cfg.K, W1, W2, cfg.dtype, **kw)
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
    return {"workload": name, "value": round(best * 1e6 * cfg.T / ntok, 1), "unit": "us", "cores": 1,
            "kind": "oracle", "sample": f"first {ntok} of {cfg.T} tokens, whole layer, 1 thread, min of 3: "
                                        f"{best:.3f} s measured, scaled x{cfg.T / ntok:g}"}


def mx_variant(steps, warmup, name="mixtral_mxfp8", iters=40):
    cfg, layer, x, r = build(name)
    ms = time_steps(layer, x, steps, warmup)
    flush = Flusher()
    fns = {"route": lambda: layer.route(x=x), "permute": lambda: layer.permute(x), "grouped_mlp": layer.mlp,
           "combine": layer.combine}
    st = {k: float(np.median(dist_cold(f, iters, flush))) for k, f in fns.items()}
    N = int(layer.offsets[-1].item())
    route_b, permute_b, combine_b, flops = algorithmic(cfg, N)
    peak = FP8_PEAK_TFLOPS if cfg.dtype == "mxfp8" else FP4_PEAK_TFLOPS
    tf = flops / (st["grouped_mlp"] * 1e-6) / 1e12
    out = {"layer_us": round(ms * 1000.0, 2), "stage_us": {k: round(v, 2) for k, v in st.items()},
           "stage_us_note": f"median of {iters} cold single calls", "grouped_gemm_tflops": round(tf, 1),
           "peak_tflops": peak, "grouped_gemm_frac_peak": round(tf / peak, 4),
           "permute_quantize_gbs": round(permute_b / (st["permute"] * 1e-6) / 1e9, 1)}
    del layer, flush
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


def other_workload(name, steps, warmup, iters=40):
    """Layer time of another full-size workload of the method (not the metric's
    configuration): the DeepSeek-like layer (256 experts, Zipf-skewed loads,
    sigmoid scores) and the sparse large-top-K share (32 of 2304 experts, K=36,
    routed from given logits with masked tokens); per stage, the median of
    `iters` cold single calls (each after a 512 MiB flush) and the warm time
    per call from graph replays."""
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
    flush = Flusher()
    fns = {"route": lambda: layer.route(x=None if logits is not None else x, logits=logits, mask=mask),
           "permute": lambda: layer.permute(x), "grouped_mlp": layer.mlp, "combine": layer.combine}
    cold = {k: float(np.median(dist_cold(f, iters, flush))) for k, f in fns.items()}
    warm = {k: float(np.median(dist_warm(f, iters, inner=2 if k == "grouped_mlp" else 8))) for k, f in fns.items()}
    mlp_us = cold["grouped_mlp"]
    out = {"workload": f"{name}: T={cfg.T} H={cfg.H} E={cfg.E} local={cfg.local} K={cfg.K} F={cfg.F}",
           "layer_us": round(us, 2), "grouped_mlp_us": round(mlp_us, 2), "routed_rows": N,
           "grouped_gemm_tflops": round(flops / (mlp_us * 1e-6) / 1e12, 1),
           "stage_us_cold": {k: round(v, 2) for k, v in cold.items()},
           "stage_us_warm": {k: round(v, 2) for k, v in warm.items()}}
    # algorithmic bytes (each token row read once, routed rows written once)
    T, H, K, E = cfg.T, cfg.H, cfg.K, cfg.E
    route_b = T * E * 4 + T * K * 6 if logits is not None else T * H * 2 + H * E * 2 + T * K * 6
    t_act = T - (T // cfg.mask_every if cfg.mask_every else 0)
    perm_b = t_act * H * 2 + N * H * 2 + T * K * 6 + N * 4
    comb_b = N * H * 2 + T * K * 8 + T * H * 2
    out["gbs_cold"] = {k: round(b / (cold[k] * 1e-6) / 1e9, 1)
                       for k, b in (("route", route_b), ("permute", perm_b), ("combine", comb_b))}
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
    else:
        # the route on plain i.i.d. N(0,1) logits (no group structure: 0.5 local routes per token)
        g = torch.Generator(device="cuda").manual_seed(5)
        plain = torch.randn((T, E), generator=g, device="cuda")
        rf = lambda: layer.route(logits=plain)
        c = float(np.median(dist_cold(rf, iters, flush)))
        w = float(np.median(dist_warm(rf, iters)))
        out["route_plain_logits_us"] = {"cold": round(c, 2), "warm": round(w, 2),
                                        "gbs_cold": round((T * E * 4 + T * K * 6) / (c * 1e-6) / 1e9, 1)}
        del plain
    del layer, x, flush
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


def pct(v):
    """median, p10 and p90 of a list of microsecond values."""
    a = np.asarray(v, np.float64)
    return {"p50": round(float(np.percentile(a, 50)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2)}


class Flusher:
    """Writes a 512 MiB buffer (the library's streaming-write calibration
    kernel): more than the 256 MB last-level cache plus the 32 MB of L2, so
    the next call finds none of its operands cached."""

    def __init__(self):
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.n = 0

    def __call__(self):
        import dropless_mixture_experts_radix_amd as D
        self.n += 1
        D.moe_calib_write(self.buf, self.n & 0xFF)


def dist_cold(fn, iters, flush):
    """GPU time of single calls of fn, each right after a cache flush (the
    flush is outside the events; the host enqueues while the flush runs)."""
    s = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in evs:
        flush()
        a.record(s)
        fn()
        b.record(s)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1000.0 for a, b in evs]


def dist_warm(fn, iters, inner=8):
    """GPU time per call of fn with its operands cached: `inner` calls back to
    back in one HIP graph, the graph replayed iters/inner times, each replay
    between two events (per-call time = replay time / inner)."""
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
    reps = max(iters // inner, 4)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    cs = torch.cuda.current_stream()
    for a, b in evs:
        a.record(cs)
        g.replay()
        b.record(cs)
    torch.cuda.synchronize()
    out = [a.elapsed_time(b) * 1000.0 / inner for a, b in evs]
    del g
    return out


def measure_ceilings():
    """Achievable rates of this GPU from the library's calibration kernels:
    streaming copy, read and write of 1 GiB, and matrix-core loops (bf16 and
    MX-scaled E4M3) on register operands; best of 5 (GB/s, TFLOP/s)."""
    import dropless_mixture_experts_radix_amd as D
    nb = 1 << 30
    src = torch.ones(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    red = torch.empty(D.moe_calib_read_out_words(nb), dtype=torch.int32, device="cuda")

    def best(fn, work, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return work / min(ts)

    out = {"copy_gbs": round(best(lambda: D.moe_calib_copy(src, dst), 2 * nb) / 1e9, 1),
           "read_gbs": round(best(lambda: D.moe_calib_read(src, red), nb) / 1e9, 1),
           "write_gbs": round(best(lambda: D.moe_calib_write(dst, 7), nb) / 1e9, 1)}
    del src, dst, red
    blocks = 256 * 4
    acc = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    for dt, key in ((D.BF16, "mfma_bf16_tflops"), (D.MXFP8, "mfma_mxfp8_tflops")):
        iters = 4096 if dt == D.BF16 else 2048
        flops = blocks * 8 * 4 * iters * (32768 if dt == D.BF16 else 131072)
        out[key] = round(best(lambda: D.moe_calib_mfma(dt, blocks, iters, acc), flops) / 1e12, 1)
    del acc
    torch.cuda.empty_cache()
    out["note"] = ("calibration kernels of the library (moe_calib_*), best of 5: copy counts bytes read + written; "
                   "matrix-core loops: 4 independent accumulators per wavefront, 8 wavefronts per CU, 4 workgroups "
                   "per CU")
    return out


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
    import dropless_mixture_experts_radix_amd as D
    calibration_copy()
    ceil = measure_ceilings()
    cfg, layer, x, r = build("mixtral_bf16")
    layer.forward(x)
    torch.cuda.synchronize()
    N = int(layer.offsets[-1].item())
    torch.cuda.synchronize()
    ms = time_steps(layer, x, a.steps, a.warmup)
    flush = Flusher()
    fns = {"route": lambda: layer.route(x=x), "permute": lambda: layer.permute(x), "grouped_mlp": layer.mlp,
           "combine": layer.combine}
    cold = {k: dist_cold(f, a.iters, flush) for k, f in fns.items()}
    warm = {k: dist_warm(f, a.iters, inner=2 if k == "grouped_mlp" else 8) for k, f in fns.items()}
    # the floor of a cold route: the library's streaming read of the same x
    # (33.5 MB), each call after the same flush
    xr = x.view(torch.uint8).reshape(-1)
    red = torch.empty(D.moe_calib_read_out_words(xr.numel()), dtype=torch.int32, device="cuda")
    read_x = dist_cold(lambda: D.moe_calib_read(xr, red), a.iters, flush)
    layer_cold = dist_cold(lambda: layer.forward(x), a.iters, flush)
    layer_warm = dist_warm(lambda: layer.forward(x), a.iters, inner=2)
    gus = time_graph(layer, x, a.steps)
    route_b, permute_b, combine_b, flops = algorithmic(cfg, N)
    med = {k: float(np.median(v)) for k, v in cold.items()}
    medw = {k: float(np.median(v)) for k, v in warm.items()}
    t_mlp = med["grouped_mlp"]  # events on the launch stream around single calls
    tflops = flops / (t_mlp * 1e-6) / 1e12
    gbs = {k: b / (med[k] * 1e-6) / 1e9 for k, b in (("route", route_b), ("permute", permute_b),
                                                     ("combine", combine_b))}
    gbs_w = {k: b / (medw[k] * 1e-6) / 1e9 for k, b in (("route", route_b), ("permute", permute_b),
                                                        ("combine", combine_b))}
    # the route reads (x, then a few bytes of ids and probs); permute and combine read and write
    ceiling_of = {"route": ceil["read_gbs"], "permute": ceil["copy_gbs"], "combine": ceil["copy_gbs"]}
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
        "stage_us": {k: round(v, 2) for k, v in med.items()},
        "stage_us_note": f"median of {a.iters} single calls, each after a 512 MiB cache flush (cold; events on "
                         f"the launch stream); stage_us_warm: HIP-graph replays of back-to-back calls",
        "stage_us_cold": {k: pct(v) for k, v in cold.items()},
        "stage_us_warm": {k: pct(v) for k, v in warm.items()},
        "layer_us_cold": pct(layer_cold),
        "layer_us_warm": pct(layer_warm),
        "graph_replay_us": round(gus, 2),
        "grouped_gemm_tflops": round(tflops, 1),
        "route_gbs": round(gbs["route"], 1),
        "permute_gbs": round(gbs["permute"], 1),
        "combine_gbs": round(gbs["combine"], 1),
        "gbs_warm": {k: round(v, 1) for k, v in gbs_w.items()},
        "frac_of_hbm_peak": {k: round(v / HBM_PEAK_GBS, 3) for k, v in gbs.items()},
        "frac_of_measured_ceiling": {**{k: round(v / ceiling_of[k], 3) for k, v in gbs.items()},
                                     "grouped_mlp": round(tflops / ceil["mfma_bf16_tflops"], 3)},
        "ceilings": ceil,
        "cold_read_x_us": pct(read_x),
        "cold_read_x_note": "the library's streaming read (moe_calib_read) of x alone, cold like the stages: the "
                            "floor under a cold route, which must read x",
        "roofline": {"kernel": "moe_grouped_mlp: k_gemm_bf16<1> (GEMM1+SwiGLU) + k_gemm_bf16<0> (GEMM2) "
                               "+ k_splitk_reduce<1,0>",
                     "bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(),
                     "traffic_unit": "HBM bytes per launch", "algorithmic_flops_per_launch": flops,
                     "time_us": round(t_mlp, 2)},
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
        line["cpu_one_core"] = [cpu_one_core("tiny_f32", 256), cpu_one_core("sparse_share", 512)]
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
