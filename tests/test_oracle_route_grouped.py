"""Pins of the oracle's group-limited routing with a selection-only bias
(oracle.route_grouped; definition: DeepSeek-V3 Technical Report, section
"DeepSeekMoE with Auxiliary-Loss-Free Load Balancing")."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "route_grouped_example.json")


def _f32_add(a, b):
    return float(np.float32(np.float32(a) + np.float32(b)))


def _brute(s_row, b_row, K, n_group, topk_group, scale):
    """Second implementation for tiny rows, by enumeration: a group's score is
    the largest fp32 sum (largest term first) over all its m-subsets; the kept
    groups are the one topk_group-subset whose every member outranks every
    other group; the selection is the one K-subset of the kept groups' experts
    whose every member outranks every other kept expert."""
    E = len(s_row)
    gs, m = E // n_group, K // topk_group
    key = [_f32_add(s_row[e], b_row[e]) for e in range(E)]
    gscore = []
    for g in range(n_group):
        best = None
        for sub in itertools.combinations(range(g * gs, (g + 1) * gs), m):
            vals = sorted((key[e] for e in sub), reverse=True)
            acc = np.float32(vals[0])
            for v in vals[1:]:
                acc = np.float32(acc + np.float32(v))
            best = float(acc) if best is None else max(best, float(acc))
        gscore.append(best)

    def g_ahead(a, b):
        return gscore[a] > gscore[b] or (gscore[a] == gscore[b] and a < b)

    kept = [G for G in itertools.combinations(range(n_group), topk_group)
            if all(g_ahead(a, b) for a in G for b in range(n_group) if b not in G)]
    assert len(kept) == 1
    allowed = [e for e in range(E) if e // gs in kept[0]]

    def e_ahead(a, b):
        return key[a] > key[b] or (key[a] == key[b] and a < b)

    sel = [S for S in itertools.combinations(allowed, K)
           if all(e_ahead(a, b) for a in S for b in allowed if b not in S)]
    assert len(sel) == 1
    ids = sorted(sel[0], key=lambda e: (-key[e], e))
    tot = sum(float(s_row[e]) for e in ids)
    return ids, [scale * float(s_row[e]) / tot for e in ids]


@pytest.mark.parametrize("E,n_group,topk_group,K", [(8, 4, 2, 4), (8, 2, 1, 2), (12, 3, 2, 4), (12, 4, 3, 3),
                                                     (8, 8, 4, 4), (12, 2, 2, 6)])
def test_matches_enumeration(E, n_group, topk_group, K):
    rng = np.random.default_rng(E * 100 + n_group * 10 + K)
    T = 40
    # few distinct values, so that equal keys and equal group scores occur
    s = rng.choice(np.array([0.125, 0.25, 0.375, 0.5, 0.625], np.float32), size=(T, E))
    bias = rng.choice(np.array([0.0, 0.0, 0.125, -0.125], np.float32), size=E)
    ids, p = O.route_grouped(None, K, n_group, topk_group, bias=bias, scale=1.5, scores=s)
    for t in range(T):
        bid, bp = _brute(s[t], bias, K, n_group, topk_group, 1.5)
        assert list(ids[t]) == bid, (t, list(ids[t]), bid)
        np.testing.assert_allclose(p[t], bp, rtol=1e-6)


def test_golden_example():
    g = json.load(open(GOLDEN))
    s = np.array([g["scores"]], np.float32)
    b = np.array(g["bias"], np.float32)
    for c in g["cases"]:
        ids, p = O.route_grouped(None, c["K"], g["n_group"], c["topk_group"], bias=b, scale=c["scale"], scores=s)
        assert list(ids[0]) == c["ids"], c["why"]
        np.testing.assert_allclose(p[0], c["probs"], rtol=1e-6)


def test_one_group_is_plain_topk():
    """n_group = topk_group = 1: every expert stays; the choice is the plain
    top-K of the keys s + b (the sort-based route oracle on those keys)."""
    rng = np.random.default_rng(7)
    z = rng.standard_normal((64, 48)).astype(np.float32)
    b = (rng.standard_normal(48) * 0.05).astype(np.float32)
    ids, _ = O.route_grouped(z, 6, 1, 1, bias=b)
    keys = (O.sigmoid_scores(z) + b[None, :]).astype(np.float32)
    want, _ = O.route_topk(keys, 6)
    np.testing.assert_array_equal(ids, want)


def test_single_expert_groups_are_plain_topk():
    """n_group = E, topk_group = K: a group's score is its one key, the K best
    groups are the K best experts."""
    rng = np.random.default_rng(8)
    z = rng.standard_normal((64, 32)).astype(np.float32)
    ids, _ = O.route_grouped(z, 4, 32, 4)
    want, _ = O.route_topk_repeated_argmax(O.sigmoid_scores(z), 4)
    np.testing.assert_array_equal(ids, want)


def test_invariants_and_selection_only_bias():
    rng = np.random.default_rng(9)
    T, E, K, ng, tg = 128, 256, 8, 8, 4
    z = rng.standard_normal((T, E)).astype(np.float32)
    b = (rng.standard_normal(E) * 0.3).astype(np.float32)
    mask = (np.arange(T) % 17 == 3).astype(np.uint8)
    ids, p = O.route_grouped(z, K, ng, tg, bias=b, scale=2.5, mask=mask)
    s = O.sigmoid_scores(z).astype(np.float64)
    live = ~mask.astype(bool)
    assert (ids[~live] == -1).all() and (p[~live] == 0).all()
    for t in np.flatnonzero(live):
        row = ids[t].astype(int)
        assert len(set(row)) == K
        assert len(set(row // (E // ng))) <= tg                      # at most topk_group groups
        np.testing.assert_allclose(p[t], 2.5 * s[t, row] / s[t, row].sum(), rtol=1e-6)  # gates: s only
    np.testing.assert_allclose(p[live].sum(axis=1), 2.5, rtol=1e-5)
    # a bias that moves no choice moves no gate
    ids0, p0 = O.route_grouped(z, K, ng, tg, bias=np.zeros(E, np.float32), scale=2.5, mask=mask)
    same = (ids0 == ids).all(axis=1)
    np.testing.assert_array_equal(p0[same], p[same])


def test_rejects_bad_shapes():
    z = np.zeros((2, 12), np.float32)
    for args in [(4, 5, 2), (4, 4, 0), (4, 4, 5), (3, 4, 2), (8, 4, 1)]:
        with pytest.raises(ValueError):
            O.route_grouped(z, *args)
