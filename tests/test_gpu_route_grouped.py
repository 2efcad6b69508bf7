"""GPU parity of the group-limited route with a selection-only bias
(moe_route_topk_grouped): sigmoid scores within a few fp32 ulps of the
float64 definition; ids bit-exact and probabilities within 1e-5 against the
oracle applied to the GPU's own fp32 scores (the choice is taken on the same
fp32 numbers); against the oracle's own scores, ids may differ only where two
keys lie within a few ulps."""
import numpy as np
import pytest
import torch

import dropless_mixture_experts_radix_amd as D
from oracle import moe_oracle as O
from tests.gpu_util import DEV, TOL, np_of, rel_inf, say, to_f64

pytestmark = pytest.mark.gpu


def _run(T, E, K, ng, tg, scale, *, logits=None, x=None, w=None, bias=None, mask=None):
    ids = torch.full((T, K), 77, dtype=torch.int16, device=DEV)
    probs = torch.full((T, K), 9.0, dtype=torch.float32, device=DEV)
    scores = torch.empty((T, E), dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    lo = ws = wp = None
    if x is not None:
        xd, wd = D.BF16, D.BF16
        wp = torch.empty(D.moe_router_prepared_bytes(x.shape[1], E, wd, xd), dtype=torch.uint8, device=DEV)
        D.moe_prepare_router(w, xd, wp)
        ws = torch.empty(max(D.moe_route_workspace_bytes(T, E, x.shape[1], xd), 16), dtype=torch.uint8, device=DEV)
        lo = torch.empty((T, E), dtype=torch.float32, device=DEV)
        D.moe_route_topk_grouped(ids, probs, ng, tg, scale, x=x, w_prepared=wp, w_dtype=wd, E=E, bias=bias,
                                 mask=mask, logits_out=lo, scores_out=scores, err=err, workspace=ws)
    else:
        D.moe_route_topk_grouped(ids, probs, ng, tg, scale, logits=logits, bias=bias, mask=mask, scores_out=scores,
                                 err=err)
    torch.cuda.synchronize()
    return np_of(ids), np_of(probs), np_of(scores), (None if lo is None else np_of(lo)), int(err.item())


def _check(ids, probs, scores, logits, K, ng, tg, scale, bias, mask):
    # scores: fp32 sigmoid within 4 ulps of the float64 definition
    want_s = 1.0 / (1.0 + np.exp(-np.asarray(logits, np.float64)))
    ulp = np.spacing(np.abs(want_s).astype(np.float32)).astype(np.float64)
    assert (np.abs(scores - want_s) <= 4 * ulp).all()
    # the choice on the GPU's own scores: bit-exact ids, probabilities 1e-5
    oi, op = O.route_grouped(logits, K, ng, tg, bias=bias, scale=scale, mask=mask, scores=scores)
    np.testing.assert_array_equal(ids, oi)
    assert rel_inf(probs, op) <= TOL["probs"]
    # against the oracle's own scores: differences only at near-ties
    oi2, _ = O.route_grouped(logits, K, ng, tg, bias=bias, scale=scale, mask=mask)
    diff = np.flatnonzero((ids != oi2).any(axis=1))
    say("  rows differing from the oracle's own sigmoid:", len(diff))
    assert len(diff) <= max(2, len(ids) // 1000)


@pytest.mark.parametrize("T,E,K,ng,tg,scale", [
    (4113, 256, 8, 8, 4, 2.5),     # the DeepSeek-V3 shape: 8 groups of 32, 4 kept, top-8
    (777, 1024, 8, 32, 4, 1.0),    # 16 keys per lane
    (300, 90, 6, 3, 3, 1.0),       # rows not 16-byte aligned, every group kept
    (500, 64, 4, 64, 4, 1.0),      # one expert per group
    (200, 128, 16, 4, 2, 1.0),     # 8 keys summed per group
    (600, 256, 8, 16, 8, 1.0),     # one key per group score, groups of 4 lanes
    (333, 512, 4, 2, 2, 1.0),      # groups of 256 experts (64 lanes)
])
def test_grouped_route_from_logits(T, E, K, ng, tg, scale):
    rng = np.random.default_rng(T + E + K)
    logits = rng.standard_normal((T, E)).astype(np.float32) * 2.0
    # Zipf-like per-expert bias (as the DeepSeek-like workload's) and masked tokens
    rank = rng.permutation(E) + 1
    bias = (-0.05 * np.log(rank)).astype(np.float32)
    mask = (np.arange(T) % 37 == 5).astype(np.uint8)
    say("grouped route", T, E, K, ng, tg)
    ids, probs, scores, _, err = _run(T, E, K, ng, tg, scale, logits=torch.from_numpy(logits).to(DEV),
                                      bias=torch.from_numpy(bias).to(DEV), mask=torch.from_numpy(mask).to(DEV))
    assert err == 0
    _check(ids, probs, scores, logits, K, ng, tg, scale, bias, mask)


def test_grouped_route_ties():
    """Few distinct logits: equal keys and equal group scores everywhere (ties
    go to the lower group and the lower expert); no bias."""
    rng = np.random.default_rng(3)
    T, E, K, ng, tg = 1000, 256, 8, 8, 4
    logits = rng.choice(np.array([-1.0, 0.0, 0.5, 1.0], np.float32), size=(T, E))
    ids, probs, scores, _, err = _run(T, E, K, ng, tg, 1.0, logits=torch.from_numpy(logits).to(DEV))
    assert err == 0
    oi, op = O.route_grouped(logits, K, ng, tg, scores=scores)
    np.testing.assert_array_equal(ids, oi)
    assert rel_inf(probs, op) <= TOL["probs"]


def test_grouped_route_from_x():
    """bf16 rows and bf16 router weights: the projection (matrix-core GEMM in
    pieces along H) feeds the grouped selection."""
    g = torch.Generator().manual_seed(11)
    T, H, E, K, ng, tg = 1500, 1024, 256, 8, 8, 4
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    w = (torch.randn((H, E), generator=g) * 0.05).to(torch.bfloat16)
    bias = (torch.randn(E, generator=g) * 0.1).float()
    ids, probs, scores, lo, err = _run(T, E, K, ng, tg, 2.5, x=x.to(DEV), w=w.to(DEV), bias=bias.to(DEV))
    assert err == 0
    want = O.router_logits(to_f64(x), to_f64(w))
    assert rel_inf(lo, want) <= TOL["logits"]
    _check(ids, probs, scores, lo, K, ng, tg, 2.5, bias.numpy(), None)


def test_grouped_route_nonfinite_logit_flags_error():
    T, E = 64, 256
    logits = np.zeros((T, E), np.float32)
    logits[5, 17] = np.inf
    _, _, _, _, err = _run(T, E, 8, 8, 4, 1.0, logits=torch.from_numpy(logits).to(DEV))
    assert err & D.DEVERR_NONFINITE
