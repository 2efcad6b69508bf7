"""Pins of the oracle's route (selection keys, top-K, probabilities).

Each check is independent of the oracle's own sort-based formula: a second
algorithm (the K repeated full-row scans the sparser-MoE page names as the
original path), brute force over all K-subsets, closed forms, and the sizes the
pages print.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from workloads import get_config
from workloads.gen import make_router_inputs, make_tokens, to_numpy_f64

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _tied_logits(rng, T, E, levels=5):
    # few distinct values -> many ties at the K-th key
    return (rng.integers(0, levels, size=(T, E)).astype(np.float32) * np.float32(0.25))


@pytest.mark.parametrize("E,K", [(8, 2), (8, 8), (33, 5), (256, 8), (300, 36), (2304, 36), (1, 1)])
@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_topk_matches_repeated_argmax(E, K, score):
    rng = np.random.default_rng(E * 131 + K)
    for logits in (rng.standard_normal((64, E)).astype(np.float32), _tied_logits(rng, 64, E)):
        bias = rng.standard_normal(E).astype(np.float32) if score == "sigmoid" else None
        a_ids, a_p = O.route_topk(logits, K, score, bias)
        b_ids, b_p = O.route_topk_repeated_argmax(logits, K, score, bias)
        np.testing.assert_array_equal(a_ids, b_ids)
        np.testing.assert_array_equal(a_p, b_p)


def _valid_topk_set(z, S):
    chosen = set(S)
    for i in chosen:
        for j in range(len(z)):
            if j in chosen:
                continue
            if not (z[i] > z[j] or (z[i] == z[j] and i < j)):
                return False
    return True


@pytest.mark.parametrize("E,K", [(4, 2), (6, 3), (8, 2), (8, 5), (7, 7)])
def test_topk_bruteforce_subsets(E, K):
    rng = np.random.default_rng(7 + E * K)
    logits = np.concatenate([_tied_logits(rng, 40, E, levels=3),
                             rng.standard_normal((40, E)).astype(np.float32)])
    ids, _ = O.route_topk(logits, K)
    for t in range(logits.shape[0]):
        z = logits[t]
        valid = [S for S in itertools.combinations(range(E), K) if _valid_topk_set(z, S)]
        assert len(valid) == 1
        assert set(ids[t].tolist()) == set(valid[0])
        # listed by descending key, ties by ascending index
        keyed = sorted(valid[0], key=lambda i: (-float(z[i]), i))
        assert ids[t].tolist() == keyed


def test_all_equal_logits_pick_lowest_ids():
    for E, K in [(8, 2), (2304, 36), (256, 8)]:
        ids, p = O.route_topk(np.zeros((3, E), np.float32), K)
        assert (ids == np.arange(K)[None, :]).all()
        np.testing.assert_allclose(p, 1.0 / K, rtol=1e-7)


def test_negative_zero_equals_positive_zero():
    logits = np.array([[-0.0, 0.0, -1.0, -0.0]], np.float32)
    ids, _ = O.route_topk(logits, 2)
    assert ids.tolist() == [[0, 1]]
    z = O.selection_keys(logits)
    assert not np.signbit(z[0, 0]) and not np.signbit(z[0, 3])


def test_nonfinite_rejected():
    with pytest.raises(ValueError):
        O.route_topk(np.array([[0.0, np.nan]], np.float32), 1)


def test_softmax_closed_form_k2():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((100, 8)).astype(np.float32)
    ids, p = O.route_topk(logits, 2)
    z0 = logits[np.arange(100), ids[:, 0]].astype(np.float64)
    z1 = logits[np.arange(100), ids[:, 1]].astype(np.float64)
    p0 = np.array([1.0 / (1.0 + math.exp(b - a)) for a, b in zip(z0, z1)])
    np.testing.assert_allclose(p[:, 0], p0, rtol=2e-7)
    np.testing.assert_allclose(p[:, 1], 1 - p0, rtol=2e-6)


def test_sigmoid_normalised_closed_form():
    # sigma(0) = 1/2, sigma(ln 3) = 3/4  ->  p = (3/4, 1/2) / (5/4) = (0.6, 0.4)
    logits = np.array([[0.0, np.float32(math.log(3.0)), -5.0]], np.float32)
    ids, p = O.route_topk(logits, 2, "sigmoid")
    assert ids.tolist() == [[1, 0]]
    np.testing.assert_allclose(p[0], [0.6, 0.4], rtol=1e-6)


def test_bias_enters_selection_and_score():
    logits = np.array([[1.0, 0.0, 0.5]], np.float32)
    bias = np.array([0.0, 2.0, 0.0], np.float32)
    ids, p = O.route_topk(logits, 1, "sigmoid", bias)
    assert ids.tolist() == [[1]]
    np.testing.assert_allclose(p, [[1.0]])


def test_probabilities_sum_to_one_and_non_increasing():
    rng = np.random.default_rng(3)
    for score in ("softmax", "sigmoid"):
        logits = rng.standard_normal((200, 300)).astype(np.float32) * 3
        _, p = O.route_topk(logits, 36, score)
        np.testing.assert_allclose(p.astype(np.float64).sum(1), 1.0, atol=1e-6)
        assert (np.diff(p.astype(np.float64), axis=1) <= 1e-7).all()


def test_mask_gives_minus_one_routes():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((10, 16)).astype(np.float32)
    mask = np.zeros(10, np.uint8)
    mask[[2, 7]] = 1
    ids, p = O.route_topk(logits, 4, mask=mask)
    assert (ids[[2, 7]] == -1).all() and (p[[2, 7]] == 0).all()
    assert (ids[[0, 1, 3]] >= 0).all()


def test_router_logits_against_python_sums():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 5)).astype(np.float32)
    w = rng.standard_normal((5, 4)).astype(np.float32)
    lg = O.router_logits(x, w)
    for t in range(3):
        for e in range(4):
            s = math.fsum(float(x[t, h]) * float(w[h, e]) for h in range(5))
            assert lg[t, e] == np.float32(s)


def test_compact_route_sizes_match_pages():
    g = json.load(open(os.path.join(GOLD, "pages_sizes.json")))
    cr = g["compact_route"]
    T, E, K = cr["T"], cr["E"], cr["K"]
    logits = np.zeros((T, 64), np.float32)  # ids storage does not depend on the values
    ids = np.zeros((T, K), np.int16)
    assert ids.nbytes == 589_824 and round(ids.nbytes / 1e6, 2) == cr["int16_ids_MB"]
    bool_map = np.zeros((T, E), np.bool_)
    assert round(bool_map.nbytes / 1e6, 2) == cr["bool_map_MB"]
    assert bool_map.nbytes // ids.nbytes == cr["ratio"]
    # the oracle's output has exactly that compact layout
    out_ids, out_p = O.route_topk(logits[:4], 36)
    assert out_ids.dtype == np.int16 and out_ids.shape == (4, 36)
    ps = g["probability_slice"]
    assert E * np.dtype(np.float32).itemsize == ps["full_row_bytes"]
    assert ps["local_experts"] * np.dtype(np.float32).itemsize == ps["local_slice_bytes"]


def test_sparse_share_workload_local_routes():
    """The large-top-K share's generator reproduces the page's 4.5 local routes
    per token and ~86% inactive local-slot checks (oracle route on a sample)."""
    g = json.load(open(os.path.join(GOLD, "pages_sizes.json")))["local_routes"]
    cfg = get_config(5)
    r = make_router_inputs(cfg, T=2048)
    ids, _ = O.route_topk(r["logits"].numpy(), cfg.K, mask=r["mask"].numpy())
    live = r["mask"].numpy() == 0
    local = ((ids >= cfg.e0) & (ids < cfg.e0 + cfg.local)).sum(1)[live]
    assert abs(local.mean() - g["local_routes_per_token"]) < 0.02 * g["local_routes_per_token"]
    inactive = 1.0 - local.mean() / g["local_experts"]
    assert abs(inactive - g["inactive_fraction"]) < 0.01
    # every selected expert lies in one of the token's 8 drawn groups
    groups = np.unique(ids[live] // 32, axis=None)
    assert (ids[live] // 32 < cfg.E // 32).all() and groups.size > 8


@pytest.mark.slow
def test_dsv3_workload_zipf_bias_empties_ten_percent():
    """The calibrated Zipf gain leaves >= 26 of 256 experts (~10%) without
    tokens and a gain 0.002 smaller does not (the calibration is a bisection to 1e-3)."""
    from workloads.configs import ZIPF_GAIN_CFG3
    from workloads.gen import zipf_bias
    cfg = get_config(3)
    x = to_numpy_f64(make_tokens(cfg))
    wr = to_numpy_f64(make_router_inputs(cfg)["w_router"])
    logits = O.router_logits(x, wr)

    def n_empty(gain):
        ids, _ = O.route_topk(logits, cfg.K, cfg.score, zipf_bias(cfg, gain).numpy())
        return int((np.bincount(ids.ravel().astype(np.int64), minlength=cfg.E) == 0).sum())

    assert n_empty(ZIPF_GAIN_CFG3) >= 26
    assert n_empty(ZIPF_GAIN_CFG3 - 0.002) < 26
