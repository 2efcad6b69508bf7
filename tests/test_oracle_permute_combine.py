"""Pins of the oracle's count/permute and combine: brute-force counting, the
stable order written out with Python loops, round-trip identities and the
degenerate cases (empty input, all -1 routes, one expert, duplicate IDs)."""
import numpy as np
import pytest

from oracle import moe_oracle as O


def _rand_ids(rng, T, K, E, p_invalid=0.1):
    ids = rng.integers(0, E, size=(T, K))
    ids[rng.random((T, K)) < p_invalid] = -1
    return ids.astype(np.int16)


@pytest.mark.parametrize("T,K,E,e0,L", [(50, 2, 8, 0, 8), (37, 36, 2304, 0, 32), (64, 8, 256, 64, 128),
                                        (1, 1, 1, 0, 1), (0, 4, 8, 0, 8), (20, 3, 5, 2, 2)])
def test_counts_offsets_order_bruteforce(T, K, E, e0, L):
    rng = np.random.default_rng(T * 7 + K)
    ids = _rand_ids(rng, T, K, E)
    x = rng.standard_normal((T, 16))
    r = O.count_and_permute(ids, e0, L, x, E_global=E)
    # counting by loops
    counts = [0] * L
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            if e0 <= e < e0 + L:
                counts[e - e0] += 1
    assert r["counts"].tolist() == counts
    assert r["offsets"][0] == 0 and r["offsets"][-1] == sum(counts)
    assert (np.diff(r["offsets"]) >= 0).all()
    # expected row order: expert by expert, then by flat index
    expect = [t * K + k for e in range(L) for t in range(T) for k in range(K) if ids[t, k] == e0 + e]
    assert r["row_to_slot"].tolist() == expect
    N = len(expect)
    for row, f in enumerate(expect):
        assert r["slot_to_row"].ravel()[f] == row
        np.testing.assert_array_equal(r["x_perm"][row], x[f // K])
    assert (r["slot_to_row"] >= 0).sum() == N


def test_duplicate_ids_in_a_token_make_two_rows():
    ids = np.array([[3, 3], [1, 3]], np.int16)
    r = O.count_and_permute(ids, 0, 4)
    assert r["counts"].tolist() == [0, 1, 0, 3]
    assert r["row_to_slot"].tolist() == [2, 0, 1, 3]


def test_single_expert_is_identity_order():
    ids = np.zeros((9, 1), np.int16)
    r = O.count_and_permute(ids, 0, 1)
    assert r["row_to_slot"].tolist() == list(range(9))


def test_out_of_range_id_rejected():
    with pytest.raises(ValueError):
        O.count_and_permute(np.array([[8]], np.int16), 0, 8, E_global=8)
    with pytest.raises(ValueError):
        O.count_and_permute(np.array([[-2]], np.int16), 0, 8, E_global=8)


def test_permute_then_combine_k1_is_identity():
    rng = np.random.default_rng(11)
    T, H, E = 40, 24, 5
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int16)
    x = rng.standard_normal((T, H))
    r = O.count_and_permute(ids, 0, E, x)
    out = O.combine(r["x_perm"], r["slot_to_row"], np.ones((T, 1), np.float32), "f64")
    np.testing.assert_array_equal(out, x)


def test_combine_all_invalid_gives_zero_rows():
    s2r = -np.ones((6, 3), np.int64)
    out = O.combine(np.zeros((0, 8)), s2r, np.ones((6, 3), np.float32), "bf16")
    assert out.shape == (6, 8) and (out == 0).all()


def test_combine_is_linear_and_weighted():
    rng = np.random.default_rng(12)
    T, K, H, N = 10, 3, 8, 40
    s2r = rng.permutation(N)[: T * K].reshape(T, K)
    s2r[0, 1] = -1
    y1, y2 = rng.standard_normal((N, H)), rng.standard_normal((N, H))
    p = rng.random((T, K)).astype(np.float32)
    a = O.combine(y1, s2r, p, "f64") + 2 * O.combine(y2, s2r, p, "f64")
    b = O.combine(y1 + 2 * y2, s2r, p, "f64")
    np.testing.assert_allclose(a, b, atol=1e-12)
    # token 0: slot 1 is skipped, the rest is a plain weighted sum
    want = float(p[0, 0]) * y1[s2r[0, 0]] + float(p[0, 2]) * y1[s2r[0, 2]]
    np.testing.assert_allclose(O.combine(y1, s2r, p, "f64")[0], want, atol=1e-12)
