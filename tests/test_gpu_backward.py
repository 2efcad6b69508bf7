"""GPU parity of the routing backward: moe_unpermute_combine_backward,
moe_permute_backward, moe_route_backward against the oracle (fp32 results
within 1e-5 of max |oracle|, bf16 within one bf16 rounding; rows and slots
without a route untouched / zero)."""
import numpy as np
import pytest
import torch

import dropless_mixture_experts_radix_amd as D
from oracle import moe_oracle as O
from tests.gpu_util import DEV, TOL, bf16_from_f64, np_of, rel_inf, say, to_f64

pytestmark = pytest.mark.gpu


def _routing(T, E, K, seed, mask_every=0, score="softmax"):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    mask = (np.arange(T) % mask_every == 1).astype(np.uint8) if mask_every else None
    ids, probs = O.route_topk(logits, K, score, mask=mask)
    perm = O.count_and_permute(ids, 0, E)
    perm["slot_to_row"] = perm["slot_to_row"].astype(np.int32)   # the library's int32 map
    return rng, logits, ids, probs, perm


def _dev_rows(v, dt):
    return bf16_from_f64(O.bf16_round(v)) if dt == "bf16" else torch.from_numpy(v.astype(np.float32)).to(DEV)


def _close_rounded(got, want, dt):
    """Each element within one rounding of the output type of the oracle's value."""
    tol = 2.0 ** -8 if dt == "bf16" else 2.0 ** -23
    assert (np.abs(got - want) <= tol * np.abs(want) + 1e-30).all()


@pytest.mark.parametrize("T,E,K,H,dt,mask_every", [
    (4096, 8, 2, 4096, "bf16", 0),      # the Mixtral-like shape
    (300, 16, 6, 64, "bf16", 7),        # masked tokens (slots without a row)
    (97, 32, 4, 200, "f32", 5),         # fp32 rows, H not a multiple of 512 values
    (1, 4, 4, 8, "bf16", 0),            # one token, the shortest row
])
def test_combine_backward(T, E, K, H, dt, mask_every):
    rng, _, ids, probs, perm = _routing(T, E, K, T + H, mask_every)
    s2r = perm["slot_to_row"]
    N = int(perm["offsets"][-1])
    cap = N + 16
    y = rng.standard_normal((cap, H))
    dout = rng.standard_normal((T, H))
    yd, gd = _dev_rows(y, dt), _dev_rows(dout, dt)
    y64, g64 = to_f64(yd), to_f64(gd)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    dy = torch.full((cap, H), 3.0, dtype=tdt, device=DEV)
    dp = torch.full((T, K), 9.0, dtype=torch.float32, device=DEV)
    say("combine backward", T, E, K, H, dt)
    D.moe_unpermute_combine_backward(gd, yd, torch.from_numpy(s2r).to(DEV), torch.from_numpy(probs).to(DEV), dy, dp)
    torch.cuda.synchronize()
    want_dy, want_dp = O.combine_backward(g64, y64, s2r, probs, "f64")
    got_dy = to_f64(dy)
    _close_rounded(got_dy[:N], want_dy, dt)
    assert (got_dy[N:] == 3.0).all()                      # rows past N untouched
    assert rel_inf(np_of(dp), want_dp) <= TOL["probs"]
    assert (np_of(dp)[s2r < 0] == 0).all()


@pytest.mark.parametrize("T,E,K,H,mask_every", [(4096, 8, 2, 4096, 0), (300, 16, 6, 96, 7), (1, 4, 4, 32, 0)])
def test_combine_backward_mx_output(T, E, K, H, mask_every):
    """The combine backward's MX output (the MXFP8 data gradient's d_y operand,
    quantized as the rows are formed): E4M3 codes and E8M0 scales bit-exact
    against the quantizer's definition applied to the bf16 d_y the same call
    writes; that bf16 d_y is the same as without the MX output; rows past N
    untouched."""
    rng, _, ids, probs, perm = _routing(T, E, K, 3 * T + H, mask_every)
    s2r = perm["slot_to_row"]
    N = int(perm["offsets"][-1])
    cap = N + 16
    # rows of very different magnitudes, so the block scales vary
    y = rng.standard_normal((cap, H))
    dout = rng.standard_normal((T, H)) * np.exp(rng.uniform(-20, 20, size=(T, 1)))
    yd, gd = _dev_rows(y, "bf16"), _dev_rows(dout, "bf16")
    s2r_d, p_d = torch.from_numpy(s2r).to(DEV), torch.from_numpy(probs).to(DEV)
    dy = torch.full((cap, H), 3.0, dtype=torch.bfloat16, device=DEV)
    dy0 = torch.full((cap, H), 3.0, dtype=torch.bfloat16, device=DEV)
    dq = torch.full((cap, H), 0x5A, dtype=torch.uint8, device=DEV)
    dqs = torch.full((cap, H // 32), 0xC3, dtype=torch.uint8, device=DEV)
    dp = torch.empty((T, K), dtype=torch.float32, device=DEV)
    say("combine backward with MX output", T, E, K, H)
    D.moe_unpermute_combine_backward(gd, yd, s2r_d, p_d, dy, dp, d_y_perm_q=dq, d_y_perm_q_scales=dqs)
    D.moe_unpermute_combine_backward(gd, yd, s2r_d, p_d, dy0, dp)
    torch.cuda.synchronize()
    got = to_f64(dy)
    np.testing.assert_array_equal(got, to_f64(dy0))
    codes, scales = O.mx_quantize_rows(got[:N])
    np.testing.assert_array_equal(np_of(dq)[:N], codes)
    np.testing.assert_array_equal(np_of(dqs)[:N], scales)
    assert (np_of(dq)[N:] == 0x5A).all() and (np_of(dqs)[N:] == 0xC3).all()


@pytest.mark.parametrize("T,E,K,H,dt,mask_every", [(4096, 8, 2, 4096, "bf16", 0), (300, 16, 6, 64, "bf16", 7),
                                                   (97, 32, 4, 200, "f32", 5)])
def test_permute_backward(T, E, K, H, dt, mask_every):
    rng, _, ids, probs, perm = _routing(T, E, K, 2 * T + H, mask_every)
    s2r = perm["slot_to_row"]
    N = int(perm["offsets"][-1])
    g = _dev_rows(rng.standard_normal((N + 8, H)), dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    dx = torch.full((T, H), 3.0, dtype=tdt, device=DEV)
    say("permute backward", T, E, K, H, dt)
    D.moe_permute_backward(g, torch.from_numpy(s2r).to(DEV), dx)
    torch.cuda.synchronize()
    want = O.permute_backward(to_f64(g), s2r, "f64")
    got = to_f64(dx)
    assert rel_inf(got, want) <= TOL[dt]
    if mask_every:
        assert (got[np.arange(T) % mask_every == 1] == 0).all()


@pytest.mark.parametrize("score,T,E,K", [("softmax", 4096, 8, 2), ("softmax", 500, 64, 8), ("sigmoid", 777, 256, 8),
                                         ("sigmoid", 50, 12, 12)])
def test_route_backward(score, T, E, K):
    rng = np.random.default_rng(T + E + K)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.2).astype(np.float32) if score == "sigmoid" else None
    mask = (np.arange(T) % 11 == 2).astype(np.uint8)
    ids, probs = O.route_topk(logits, K, score, bias=bias, mask=mask)
    g = rng.standard_normal((T, K)).astype(np.float32)
    dz = torch.full((T, K), 9.0, dtype=torch.float32, device=DEV)
    code = D.SOFTMAX if score == "softmax" else D.SIGMOID
    say("route backward", score, T, E, K)
    D.moe_route_backward(torch.from_numpy(ids).to(DEV), torch.from_numpy(g).to(DEV), dz, code,
                         probs=torch.from_numpy(probs).to(DEV), logits=torch.from_numpy(logits).to(DEV),
                         score_bias=None if bias is None else torch.from_numpy(bias).to(DEV), E=E)
    torch.cuda.synchronize()
    want = O.route_backward(ids, g, score, probs=probs, logits=logits, score_bias=bias)
    assert rel_inf(np_of(dz), want) <= TOL["probs"]
    assert (np_of(dz)[mask.astype(bool)] == 0).all()


def test_route_backward_grouped_gates():
    """The group-limited route's gates: scale 2.5, no bias in the scores."""
    rng = np.random.default_rng(5)
    T, E, K = 1000, 256, 8
    logits = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    ids, probs = O.route_grouped(logits, K, 8, 4, bias=bias, scale=2.5)
    g = rng.standard_normal((T, K)).astype(np.float32)
    dz = torch.empty((T, K), dtype=torch.float32, device=DEV)
    D.moe_route_backward(torch.from_numpy(ids).to(DEV), torch.from_numpy(g).to(DEV), dz, D.SIGMOID,
                         logits=torch.from_numpy(logits).to(DEV), scale=2.5)
    torch.cuda.synchronize()
    want = O.route_backward(ids, g, "sigmoid", logits=logits, scale=2.5)
    assert rel_inf(np_of(dz), want) <= TOL["probs"]
