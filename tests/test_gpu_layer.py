"""GPU parity of the whole layer (route -> permute -> grouped MLP -> combine)
on the workloads, in the configuration the benchmark times, plus HIP-graph
capture and replay on new data (nothing in the layer needs the host).

Small workloads are compared element by element with the oracle.  The large
ones are checked on every token for the integer parts (ids, counts, offsets,
maps, permuted rows) and on sampled rows/tokens for the float parts, which the
oracle computes one by one."""
import numpy as np
import pytest
import torch

import dropless_mixture_experts_radix_amd as D
from dropless_mixture_experts_radix_amd import MoELayer
from oracle import moe_oracle as O
from tests.gpu_util import DEV, TOL, np_of, rel_inf, say, to_f64
from workloads import get_config
from workloads.gen import make_expert_weights, make_router_inputs, make_tokens, to_numpy_f64

pytestmark = pytest.mark.gpu

DT = {"f32": D.F32, "bf16": D.BF16, "mxfp8": D.MXFP8, "mxfp4": D.MXFP4}


def build_layer(cfg, keep=(), T=None):
    T = cfg.T if T is None else T
    x = make_tokens(cfg, T=T).to(DEV)
    r = make_router_inputs(cfg, T=T)
    layer = MoELayer(T, cfg.H, cfg.E, cfg.K, cfg.F, DT[cfg.dtype], DT[cfg.x_dtype], L=cfg.local, e0=cfg.e0,
                     score=D.SIGMOID if cfg.score == "sigmoid" else D.SOFTMAX,
                     w_router=None if r["w_router"] is None else r["w_router"].to(DEV),
                     bias=None if r["bias"] is None else r["bias"].to(DEV))
    kept = {}
    for e in range(cfg.local):
        w1, w2 = make_expert_weights(cfg, cfg.e0 + e, device=DEV)
        layer.set_expert_weights(e, w1, w2)
        if keep == "all" or e in keep:
            kept[e] = (w1, w2)
        del w1, w2
    logits = None if r["logits"] is None else r["logits"].to(DEV)
    mask = None if r["mask"] is None else r["mask"].to(DEV)
    return layer, x, r, logits, mask, kept


def run(layer, x, logits, mask):
    out = layer.forward(x, logits=logits, mask=mask, write_logits=True)
    torch.cuda.synchronize()
    return out


def check_route_and_permute(cfg, layer, x, r):
    """Every token: ids/probs against the oracle on the GPU logits, and the
    whole count/permute against the oracle on the GPU ids."""
    lo = np_of(layer.logits_out)
    bias = None if r["bias"] is None else r["bias"].numpy()
    mask = None if r["mask"] is None else r["mask"].numpy()
    o_ids, o_p = O.route_topk(lo, cfg.K, cfg.score, bias, mask)
    ids = np_of(layer.ids)
    np.testing.assert_array_equal(ids, o_ids)
    assert rel_inf(np_of(layer.probs), o_p) <= TOL["probs"]
    ref = O.count_and_permute(ids, cfg.e0, cfg.local, None, E_global=cfg.E)
    N = int(ref["offsets"][-1])
    np.testing.assert_array_equal(np_of(layer.counts), ref["counts"])
    np.testing.assert_array_equal(np_of(layer.offsets), ref["offsets"])
    np.testing.assert_array_equal(np_of(layer.row_to_slot)[:N], ref["row_to_slot"])
    np.testing.assert_array_equal(np_of(layer.slot_to_row), ref["slot_to_row"])
    assert int(layer.err.item()) == 0
    return ref, N


@pytest.mark.parametrize("name", ["micro", "tiny_f32"])
def test_layer_small_workloads_full_oracle(name):
    cfg = get_config(name)
    say("layer", name)
    layer, x, r, logits, mask, kept = build_layer(cfg, keep="all")
    out = run(layer, x, logits, mask)
    ref, N = check_route_and_permute(cfg, layer, x, r)
    W1 = [to_numpy_f64(kept[e][0]) for e in range(cfg.local)]
    W2 = [to_numpy_f64(kept[e][1]) for e in range(cfg.local)]
    want = O.layer(to_f64(x), cfg.K, W1, W2, cfg.dtype, logits=np_of(layer.logits_out), score=cfg.score)
    # the projection against its float64 definition
    assert rel_inf(np_of(layer.logits_out), O.router_logits(to_f64(x), to_numpy_f64(r["w_router"]))) <= TOL["logits"]
    np.testing.assert_array_equal(to_f64(layer.x_perm)[:N], want["x_perm"])
    assert rel_inf(to_f64(layer.y_perm)[:N], want["y_perm"]) <= TOL[cfg.dtype]
    assert rel_inf(to_f64(out), want["out"]) <= TOL[cfg.dtype]


def test_layer_sparse_share_full_oracle():
    """The large-top-K share (T=8192, E=2304, K=36, 32 local experts, H=F=512),
    whole layer against the oracle on every element."""
    cfg = get_config("sparse_share")
    say("layer sparse_share full")
    layer, x, r, logits, mask, kept = build_layer(cfg, keep="all")
    out = run(layer, x, logits, mask)
    ref, N = check_route_and_permute(cfg, layer, x, r)
    W1 = [to_numpy_f64(kept[e][0]) for e in range(cfg.local)]
    W2 = [to_numpy_f64(kept[e][1]) for e in range(cfg.local)]
    want = O.layer(to_f64(x), cfg.K, W1, W2, "bf16", logits=r["logits"].numpy(), mask=r["mask"].numpy(),
                   e0=cfg.e0, L=cfg.local)
    np.testing.assert_array_equal(to_f64(layer.x_perm)[:N], want["x_perm"])
    assert rel_inf(to_f64(layer.y_perm)[:N], want["y_perm"]) <= TOL["bf16"]
    assert rel_inf(to_f64(out), want["out"]) <= TOL["bf16"]
    masked = r["mask"].numpy() == 1
    assert (to_f64(out)[masked] == 0).all()


def _sampled_expert_rows(offsets, experts, per=6, seed=0):
    rng = np.random.default_rng(seed)
    rows = {}
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        pick = {lo, hi - 1} | set(rng.integers(lo, hi, size=per).tolist())
        rows[e] = sorted(pick)
    return rows


@pytest.mark.parametrize("name", ["mixtral_bf16", "mixtral_mxfp8", "mixtral_mxfp4", "dsv3_bf16"])
def test_layer_large_workloads_sampled(name):
    cfg = get_config(name)
    say("layer", name, "full size, sampled float checks")
    layer, x, r, logits, mask, _ = build_layer(cfg, keep=())
    out = run(layer, x, logits, mask)
    ref, N = check_route_and_permute(cfg, layer, x, r)
    # projection on sampled tokens
    rows_t = np.linspace(0, cfg.T - 1, 256).astype(int)
    want_lo = O.router_logits(to_f64(x[rows_t]), to_numpy_f64(r["w_router"]))
    assert rel_inf(np_of(layer.logits_out)[rows_t], want_lo) <= TOL["logits"]
    # permuted rows: every row against the token row it came from
    r2s = layer.row_to_slot[:N].long()
    src = x[r2s // cfg.K]
    if cfg.dtype == "mxfp8":
        sample = np.linspace(0, N - 1, 512).astype(int)
        c, s = O.mx_quantize_rows(to_f64(src[sample]))
        np.testing.assert_array_equal(np_of(layer.x_perm[sample]), c)
        np.testing.assert_array_equal(np_of(layer.x_perm_scales[sample]), s)
    elif cfg.dtype == "mxfp4":
        sample = np.linspace(0, N - 1, 512).astype(int)
        c, s = O.mx4_quantize_rows(to_f64(src[sample]))
        np.testing.assert_array_equal(np_of(layer.x_perm[sample]), O.pack_fp4(c))
        np.testing.assert_array_equal(np_of(layer.x_perm_scales[sample]), s)
    else:
        assert torch.equal(layer.x_perm[:N], src)
    # grouped MLP on sampled rows of sampled experts (largest, smallest non-empty, one more)
    counts = ref["counts"]
    nz = np.flatnonzero(counts)
    experts = sorted({int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])]), int(nz[len(nz) // 2])})
    if cfg.E <= 8:
        experts = experts[:2]
    rows = _sampled_expert_rows(ref["offsets"], experts)
    for e, rr in rows.items():
        w1, w2 = make_expert_weights(cfg, cfg.e0 + e, device=DEV)
        W1, W2 = to_numpy_f64(w1), to_numpy_f64(w2)
        del w1, w2
        X = to_f64(x[r2s[rr] // cfg.K])
        want_y, _ = O.expert_mlp(X, W1, W2, cfg.dtype)
        err = rel_inf(to_f64(layer.y_perm[torch.tensor(rr, device=DEV)]), want_y)
        say("  expert", e, "rows", len(rr), "rel", err)
        assert err <= TOL[cfg.dtype]
        del W1, W2
    # combine on sampled tokens, from the GPU's expert rows
    toks = np.linspace(0, cfg.T - 1, 64).astype(int)
    s2r = np_of(layer.slot_to_row)[toks]
    used = np.unique(s2r[s2r >= 0])
    yp = to_f64(layer.y_perm[torch.from_numpy(used).to(DEV)])
    s2r_c = np.where(s2r >= 0, np.searchsorted(used, s2r), -1)
    want_out = O.combine(yp, s2r_c, np_of(layer.probs)[toks], "bf16")
    assert rel_inf(to_f64(out)[toks], want_out) <= TOL[cfg.dtype]


def test_layer_graph_capture_replays_on_new_data():
    cfg = get_config("sparse_share")
    T = 1024
    say("graph capture")
    layer, x, r, logits, mask, _ = build_layer(cfg, T=T)
    static_x = x.clone()
    static_logits = logits.clone()
    run(layer, static_x, static_logits, mask)  # warm up outside capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        layer.forward(static_x, logits=static_logits, mask=mask)
    torch.cuda.synchronize()
    gen = torch.Generator(device=DEV)
    for rep in range(3):
        gen.manual_seed(100 + rep)
        static_x.copy_(torch.randn(static_x.shape, generator=gen, device=DEV).to(static_x.dtype))
        static_logits.copy_(torch.randn(static_logits.shape, generator=gen, device=DEV) +
                            16.0 * (torch.rand(static_logits.shape, generator=gen, device=DEV) < 0.1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = layer.out.clone()
        got_ids = layer.ids.clone()
        layer.forward(static_x, logits=static_logits, mask=mask)  # eager on the same data
        torch.cuda.synchronize()
        assert torch.equal(got_ids, layer.ids)
        assert torch.equal(got, layer.out)
