"""Pins of the oracle's grouped SwiGLU MLP and whole layer: an explicit Python
triple loop on a micro layer, torch's dense MLP (an independent library) for
the one-expert and identical-experts reductions, empty experts, and the MXFP8
path on values already on the MX grid (where quantization is the identity)."""
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import get_config
from workloads.gen import make_expert_weights, make_router_inputs, make_tokens, to_numpy_f64


def _micro():
    cfg = get_config("micro")
    x = to_numpy_f64(make_tokens(cfg))
    r = make_router_inputs(cfg)
    W = [make_expert_weights(cfg, e) for e in range(cfg.E)]
    W1 = [to_numpy_f64(w[0]) for w in W]
    W2 = [to_numpy_f64(w[1]) for w in W]
    return cfg, x, to_numpy_f64(r["w_router"]), W1, W2


def test_micro_layer_against_python_loops():
    cfg, x, wr, W1, W2 = _micro()
    res = O.layer(x, cfg.K, W1, W2, "f64", w_router=wr)
    T, H, F, K = cfg.T, cfg.H, cfg.F, cfg.K
    for t in range(T):
        acc = [0.0] * H
        for k in range(K):
            e = int(res["ids"][t, k])
            p = float(res["probs"][t, k])
            h = [math.fsum(x[t, i] * W1[e][i, j] for i in range(H)) for j in range(2 * F)]
            a = [h[j] / (1.0 + math.exp(-h[j])) * h[F + j] for j in range(F)]
            y = [math.fsum(a[j] * W2[e][j, c] for j in range(F)) for c in range(H)]
            for c in range(H):
                acc[c] += p * y[c]
        np.testing.assert_allclose(res["out"][t], acc, rtol=1e-12, atol=1e-14)


def _torch_dense(x, w1, w2, F):
    xt, a1, a2 = (torch.from_numpy(np.asarray(v, np.float64)) for v in (x, w1, w2))
    h = xt @ a1
    return (torch.nn.functional.silu(h[:, :F]) * h[:, F:]) @ a2


def test_single_expert_is_dense_mlp():
    rng = np.random.default_rng(1)
    T, H, F = 17, 32, 48
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((H, 2 * F)) * 0.2
    w2 = rng.standard_normal((F, H)) * 0.2
    ids = np.zeros((T, 1), np.int16)
    perm = O.count_and_permute(ids, 0, 1, x)
    y, _ = O.grouped_mlp(perm["x_perm"], perm["offsets"], [w1], [w2], "f64")
    np.testing.assert_allclose(y, _torch_dense(x, w1, w2, F).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_identical_experts_layer_is_dense_mlp(score):
    rng = np.random.default_rng(2)
    T, H, F, E, K = 40, 32, 64, 6, 3
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((H, 2 * F)) * 0.2
    w2 = rng.standard_normal((F, H)) * 0.2
    logits = rng.standard_normal((T, E)).astype(np.float32)
    res = O.layer(x, K, [w1] * E, [w2] * E, "f64", logits=logits, score=score)
    # probabilities are fp32, their sum is 1 within fp32 rounding
    want = _torch_dense(x, w1, w2, F).numpy() * res["probs"].astype(np.float64).sum(1, keepdims=True)
    np.testing.assert_allclose(res["out"], want, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(res["probs"].astype(np.float64).sum(1), 1.0, atol=1e-6)


def test_empty_experts_produce_no_rows():
    rng = np.random.default_rng(3)
    T, H, F, E = 12, 32, 32, 5
    x = rng.standard_normal((T, H))
    ids = np.where(rng.random((T, 2)) < 0.5, 1, 3).astype(np.int16)
    W1 = [None, rng.standard_normal((H, 2 * F)), None, rng.standard_normal((H, 2 * F)), None]
    W2 = [None, rng.standard_normal((F, H)), None, rng.standard_normal((F, H)), None]
    perm = O.count_and_permute(ids, 0, E, x)
    assert perm["counts"][[0, 2, 4]].tolist() == [0, 0, 0]
    y, _ = O.grouped_mlp(perm["x_perm"], perm["offsets"], W1, W2, "f64")  # W[e]=None never touched
    assert y.shape == (T * 2, H)


def test_all_routes_invalid_layer_gives_zeros():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 32))
    logits = rng.standard_normal((6, 4)).astype(np.float32)
    res = O.layer(x, 2, [None] * 4, [None] * 4, "bf16", logits=logits, mask=np.ones(6, np.uint8))
    assert (res["out"] == 0).all() and res["offsets"][-1] == 0


def test_mxfp8_on_grid_values_equals_unquantized_path():
    """Inputs whose every 32-block already lies on the E4M3 grid at its own MX
    scale quantize exactly; the MXFP8 expert MLP then equals the bf16 one fed
    the same values except for the quantization of `a`."""
    rng = np.random.default_rng(5)
    grid = O.e4m3_decode(np.arange(0x30, 0x7F, dtype=np.uint8))  # 0.5 .. 448

    def on_grid(shape):
        v = rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        v.reshape(-1, 32)[:, 0] = 448.0  # fix every block's scale at 2^0
        return v

    T, H, F = 8, 64, 64
    x = on_grid((T, H)) * 2.0 ** -8
    w1 = on_grid((2 * F, H)).T * 2.0 ** -12
    w2 = on_grid((H, F)).T * 2.0 ** -12
    for m in (x, w1.T, w2.T):
        c, s = O.mx_quantize_rows(m)
        np.testing.assert_array_equal(O.mx_dequantize_rows(c, s), m)
    y_mx, a_mx = O.expert_mlp(x, w1, w2, "mxfp8")
    h = x @ w1
    a = O.bf16_round(O.swiglu(h, F))
    np.testing.assert_array_equal(a_mx, a)
    aq = O.mx_dequantize_rows(*O.mx_quantize_rows(a))
    np.testing.assert_array_equal(y_mx, O.bf16_round(aq @ w2))


def test_mxfp4_on_grid_values_equals_unquantized_path():
    """Inputs whose every 32-block lies on the E2M1 grid at its own MX scale
    quantize exactly; the MXFP4 expert MLP then equals the bf16 one fed the
    same values except for the quantization of `a`."""
    rng = np.random.default_rng(6)
    grid = O.e2m1_decode(np.arange(1, 8, dtype=np.uint8))  # 0.5 .. 6

    def on_grid(shape):
        v = rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        v.reshape(-1, 32)[:, 0] = 6.0  # fix every block's scale at 2^0
        return v

    T, H, F = 8, 64, 64
    x = on_grid((T, H)) * 2.0 ** -3
    w1 = on_grid((2 * F, H)).T * 2.0 ** -6
    w2 = on_grid((H, F)).T * 2.0 ** -6
    for m in (x, w1.T, w2.T):
        c, s = O.mx4_quantize_rows(m)
        np.testing.assert_array_equal(O.mx4_dequantize_rows(c, s), m)
    y_mx, a_mx = O.expert_mlp(x, w1, w2, "mxfp4")
    h = x @ w1
    a = O.bf16_round(O.swiglu(h, F))
    np.testing.assert_array_equal(a_mx, a)
    aq = O.mx4_dequantize_rows(*O.mx4_quantize_rows(a))
    np.testing.assert_array_equal(y_mx, O.bf16_round(aq @ w2))
    # the quantized activations differ from the exact ones by at most half a
    # step of their block
    assert np.abs(aq - a).max() <= np.abs(a).max() / 4
