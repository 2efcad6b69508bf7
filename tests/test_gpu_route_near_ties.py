"""End-to-end route selection against the oracle's own float64 logits.

The parity tests hold the GPU's ids to the oracle applied to the GPU's fp32
logits.  Here the ids come from the original inputs and are compared with the
selection the oracle makes on its float64 projection of the same x and router
weights.  The two projections differ by summation order and rounding, so a
token may select differently only where its keys are nearly tied: a different
set of experts is allowed when the oracle's K-th and (K+1)-th keys are within
4 fp32 ulps, the same set in another order when the two swapped keys are.
Every such case is counted and printed (expected about zero); any other
mismatch fails.  Selection keys are logit + bias, the reading the route
kernels and the oracle share."""
import numpy as np
import pytest
import torch

import dropless_mixture_experts_radix_amd as D
from dropless_mixture_experts_radix_amd import MoELayer
from oracle import moe_oracle as O
from tests.gpu_util import DEV, np_of, say, to_f64
from workloads import get_config
from workloads.gen import make_router_inputs, make_tokens, to_numpy_f64

pytestmark = pytest.mark.gpu

DT = {"f32": D.F32, "bf16": D.BF16, "mxfp8": D.MXFP8, "mxfp4": D.MXFP4}
ULPS = 4


def near(a, b):
    """|a - b| within ULPS fp32 ulps of the larger magnitude."""
    m = np.maximum(np.abs(a), np.abs(b)).astype(np.float32)
    return np.abs(a - b) <= ULPS * np.spacing(m).astype(np.float64)


def classify(ids, o_ids, z, K):
    """Mismatching tokens: (near-tie set mismatches, near-tie order swaps, other)."""
    near_set = near_order = other = 0
    bad = np.nonzero((ids != o_ids).any(axis=1))[0]
    for t in bad:
        keys = np.sort(z[t])[::-1]
        if set(ids[t].tolist()) != set(o_ids[t].tolist()):
            if K < z.shape[1] and near(keys[K - 1], keys[K]):
                near_set += 1
            else:
                other += 1
        else:
            # same experts, another order: every swapped pair of keys must be tied
            ok = all(near(z[t, a], z[t, b]) for a, b in zip(ids[t], o_ids[t]) if a != b)
            if ok:
                near_order += 1
            else:
                other += 1
    return near_set, near_order, other


@pytest.mark.parametrize("name", ["tiny_f32", "mixtral_bf16", "dsv3_bf16"])
def test_route_ids_against_float64_logits(name):
    cfg = get_config(name)
    say("near ties", name)
    x = make_tokens(cfg).to(DEV)
    r = make_router_inputs(cfg)
    layer = MoELayer(cfg.T, cfg.H, cfg.E, cfg.K, cfg.F, DT[cfg.dtype], DT[cfg.x_dtype], L=cfg.local, e0=cfg.e0,
                     score=D.SIGMOID if cfg.score == "sigmoid" else D.SOFTMAX,
                     w_router=r["w_router"].to(DEV), bias=None if r["bias"] is None else r["bias"].to(DEV))
    layer.route(x=x)
    torch.cuda.synchronize()
    ids = np_of(layer.ids).astype(np.int64)
    logits = O.router_logits(to_f64(x), to_numpy_f64(r["w_router"]))
    bias = None if r["bias"] is None else r["bias"].numpy()
    o_ids, _ = O.route_topk(logits, cfg.K, cfg.score, bias)
    z = O.selection_keys(logits, bias).astype(np.float64)
    near_set, near_order, other = classify(ids, o_ids.astype(np.int64), z, cfg.K)
    say(f"  {name}: {cfg.T} tokens, near-tie set mismatches {near_set}, near-tie order swaps {near_order}, "
        f"other mismatches {other}")
    assert other == 0
