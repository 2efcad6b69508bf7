"""Randomised small-shape sweep of the whole layer on the GPU (Hypothesis).

Shapes are drawn from T in {0, 1, 3, 257}, E in {1, 2, 8, 33, 300}, K <= E,
H in {32, 96}, with a random slice of local experts (e0, L), either score
function and an optional per-expert bias.  Every example runs route ->
count/permute -> grouped MLP -> combine in fp32 and is compared with the
oracle: the selection on the GPU's own logits (ids exact, probabilities to
1e-5), the counts, offsets, maps and permuted rows bit for bit, the MLP and
the combined output to 1e-5.  The same ids then permute bf16 rows, compared
bit for bit as well.  The draw is derandomised, so the examples are the same
on every run; each one prints its case before it starts."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import dropless_mixture_experts_radix_amd as D
from dropless_mixture_experts_radix_amd import MoELayer
from oracle import moe_oracle as O
from tests.gpu_util import DEV, TOL, bf16_from_f64, np_of, rel_inf, say, to_f64

pytestmark = pytest.mark.gpu


@st.composite
def shapes(draw):
    T = draw(st.sampled_from([0, 1, 3, 257]))
    E = draw(st.sampled_from([1, 2, 8, 33, 300]))
    K = draw(st.integers(1, min(E, 64)))  # at most 64 routes per token (the library limit)
    H = draw(st.sampled_from([32, 96]))
    F = draw(st.sampled_from([32, 64]))
    e0 = draw(st.integers(0, E - 1))
    L = draw(st.integers(1, E - e0))
    score = draw(st.sampled_from(["softmax", "sigmoid"]))
    biased = draw(st.booleans())
    seed = draw(st.integers(0, 2**31 - 1))
    return T, E, K, H, F, e0, L, score, biased, seed


@settings(max_examples=60, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(shapes())
def test_layer_small_shapes_sweep(case):
    T, E, K, H, F, e0, L, score, biased, seed = case
    say("sweep", dict(T=T, E=E, K=K, H=H, F=F, e0=e0, L=L, score=score, biased=biased, seed=seed))
    rng = np.random.default_rng(seed)
    x64 = rng.standard_normal((T, H)).astype(np.float32).astype(np.float64)
    wr64 = (rng.standard_normal((H, E)) * 0.3).astype(np.float32).astype(np.float64)
    bias = (rng.standard_normal(E) * 0.5).astype(np.float32) if biased else None
    W1 = [(rng.standard_normal((H, 2 * F)) * 0.2).astype(np.float32).astype(np.float64) for _ in range(L)]
    W2 = [(rng.standard_normal((F, H)) * 0.2).astype(np.float32).astype(np.float64) for _ in range(L)]
    x = torch.from_numpy(x64.astype(np.float32)).to(DEV)
    layer = MoELayer(T, H, E, K, F, D.F32, D.F32, L=L, e0=e0,
                     score=D.SIGMOID if score == "sigmoid" else D.SOFTMAX,
                     w_router=torch.from_numpy(wr64.astype(np.float32)).to(DEV),
                     bias=None if bias is None else torch.from_numpy(bias).to(DEV))
    for e in range(L):
        layer.set_expert_weights(e, torch.from_numpy(W1[e].astype(np.float32)).to(DEV),
                                 torch.from_numpy(W2[e].astype(np.float32)).to(DEV))
    out = layer.forward(x, write_logits=True)
    torch.cuda.synchronize()
    assert int(layer.err.item()) == 0
    lo = np_of(layer.logits_out).astype(np.float64)
    assert rel_inf(lo, O.router_logits(x64, wr64)) <= TOL["logits"]
    o_ids, o_p = O.route_topk(lo, K, score, bias)
    ids = np_of(layer.ids)
    np.testing.assert_array_equal(ids, o_ids)
    assert rel_inf(np_of(layer.probs), o_p) <= TOL["probs"]
    want = O.layer(x64, K, W1, W2, "f32", logits=lo, score=score, bias=bias, e0=e0, L=L)
    N = int(want["offsets"][-1])
    np.testing.assert_array_equal(np_of(layer.counts), want["counts"])
    np.testing.assert_array_equal(np_of(layer.offsets), want["offsets"])
    np.testing.assert_array_equal(np_of(layer.row_to_slot)[:N], want["row_to_slot"])
    np.testing.assert_array_equal(np_of(layer.slot_to_row), want["slot_to_row"])
    np.testing.assert_array_equal(to_f64(layer.x_perm)[:N], want["x_perm"])
    assert rel_inf(to_f64(layer.y_perm)[:N], want["y_perm"]) <= TOL["f32"]
    assert rel_inf(to_f64(out), want["out"]) <= TOL["f32"]
    # the same ids permute bf16 rows, bit for bit
    xb64 = O.bf16_round(x64)
    ref = O.count_and_permute(ids, e0, L, xb64, E_global=E)
    cap = max(T * min(K, L), 1)
    counts = torch.empty(L, dtype=torch.int32, device=DEV)
    offsets = torch.empty(L + 1, dtype=torch.int32, device=DEV)
    xp = torch.full((cap, H), 5.0, dtype=torch.bfloat16, device=DEV)
    r2s = torch.full((cap,), -7, dtype=torch.int32, device=DEV)
    s2r = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    ws = torch.zeros(D.moe_permute_workspace_bytes(T, K, L), dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    D.moe_permute(bf16_from_f64(xb64), torch.from_numpy(ids).to(DEV), E, e0, L, counts, offsets, xp, r2s, s2r, ws,
                  err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    np.testing.assert_array_equal(np_of(offsets), ref["offsets"])
    np.testing.assert_array_equal(np_of(s2r), ref["slot_to_row"])
    np.testing.assert_array_equal(np_of(r2s)[:N], ref["row_to_slot"])
    np.testing.assert_array_equal(to_f64(xp)[:N], ref["x_perm"])
