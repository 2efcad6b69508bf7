"""GPU parity: MX quantizer (bit-exact) and route (projection within 1e-5,
ids bit-exact and probabilities within 1e-5 against the oracle applied to the
GPU's own logits)."""
import numpy as np
import pytest
import torch

import dropless_mixture_experts_radix_amd as D
from oracle import moe_oracle as O
from tests.gpu_util import DEV, TOL, bf16_from_bits, bf16_from_f64, np_of, rel_inf, say, to_f64
from workloads import get_config
from workloads.gen import make_router_inputs, make_tokens, to_numpy_f64

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------- MX
def _mx_gpu(x_bf16, row_limit=None, sentinel=None):
    rows, cols = x_bf16.shape
    codes = torch.full((rows, cols), 0xAB if sentinel is None else sentinel, dtype=torch.uint8, device=DEV)
    scales = torch.full((rows, cols // 32), 0xCD, dtype=torch.uint8, device=DEV)
    D.moe_mx_quantize(x_bf16, codes, scales, row_limit)
    torch.cuda.synchronize()
    return np_of(codes), np_of(scales)


def test_mx_quantize_every_bf16_pattern_as_block_max():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = O.bits_to_bf16(bits)
    keep = np.isfinite(vals)
    bits = bits[keep]
    blocks = np.zeros((bits.size, 32), np.uint16)
    blocks[:, 5] = bits
    blocks[:, 6] = bits ^ 0x8000           # the negated value
    blocks[:, 7] = (bits & 0x7fff) >> 1    # a smaller-magnitude neighbour
    blocks[:, 9] = 0x8000                  # -0.0
    say("mx exhaustive: blocks", blocks.shape)
    codes, scales = _mx_gpu(bf16_from_bits(blocks))
    oc, os_ = O.mx_quantize_rows(O.bits_to_bf16(blocks))
    np.testing.assert_array_equal(scales, os_)
    np.testing.assert_array_equal(codes, oc)


def test_mx_quantize_random_wide_range_and_row_limit():
    rng = np.random.default_rng(5)
    raw = rng.standard_normal((3000, 256)) * np.exp(rng.uniform(-40, 40, size=(3000, 1)))
    raw[::7, :32] = 0.0
    v = O.bf16_round(raw)
    x = bf16_from_f64(v)
    lim = torch.tensor([2500], dtype=torch.int32, device=DEV)
    codes, scales = _mx_gpu(x, row_limit=lim, sentinel=0x5A)
    oc, os_ = O.mx_quantize_rows(v[:2500])
    np.testing.assert_array_equal(codes[:2500], oc)
    np.testing.assert_array_equal(scales[:2500], os_)
    assert (codes[2500:] == 0x5A).all() and (scales[2500:] == 0xCD).all()


# --------------------------------------------------------------------------- route
def _route_gpu(T, E, K, score, *, logits=None, x=None, w_router=None, bias=None, mask=None):
    layer_ids = torch.empty((T, K), dtype=torch.int16, device=DEV)
    probs = torch.empty((T, K), dtype=torch.float32, device=DEV)
    lo = torch.full((T, E), float("nan"), dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kw = dict(bias=bias, mask=mask, logits_out=lo, err=err)
    if logits is not None:
        D.moe_route_topk(layer_ids, probs, score, logits=logits, **kw)
    else:
        xd = D._lib.dtype_code(x.dtype)
        wd = D._lib.dtype_code(w_router.dtype)
        wp = torch.empty(D.moe_router_prepared_bytes(x.shape[1], E, wd, xd), dtype=torch.uint8, device=DEV)
        D.moe_prepare_router(w_router, xd, wp)
        ws = torch.empty(max(D.moe_route_workspace_bytes(T, E, x.shape[1], xd), 16), dtype=torch.uint8, device=DEV)
        D.moe_route_topk(layer_ids, probs, score, x=x, w_prepared=wp, w_dtype=wd, E=E, workspace=ws, **kw)
    torch.cuda.synchronize()
    return np_of(layer_ids), np_of(probs), np_of(lo), int(err.item())


def _check_route(ids, probs, lo, T, K, score, bias=None, mask=None):
    o_ids, o_p = O.route_topk(lo, K, score, bias, mask)
    np.testing.assert_array_equal(ids, o_ids)
    assert rel_inf(probs, o_p) <= TOL["probs"]


@pytest.mark.parametrize("cfgname,T", [("tiny_f32", 256), ("mixtral_bf16", 1024), ("mixtral_bf16", 4096),
                                       ("mixtral_bf16", 1000), ("mixtral_bf16", 4113), ("dsv3_bf16", 1024),
                                       ("dsv3_bf16", 8192)])
def test_route_fused_projection_workloads(cfgname, T):
    cfg = get_config(cfgname)
    say("route", cfgname, T)
    x = make_tokens(cfg, T=T)
    r = make_router_inputs(cfg, T=T)
    bias = None if r["bias"] is None else r["bias"].to(DEV)
    score = D.SIGMOID if cfg.score == "sigmoid" else D.SOFTMAX
    ids, probs, lo, err = _route_gpu(T, cfg.E, cfg.K, score, x=x.to(DEV), w_router=r["w_router"].to(DEV), bias=bias)
    assert err == 0
    # projection against the float64 definition (sampled rows for the large shapes)
    rows = np.arange(T) if T <= 1024 else np.linspace(0, T - 1, 512).astype(int)
    want = O.router_logits(to_numpy_f64(x[rows]), to_numpy_f64(r["w_router"]))
    assert rel_inf(lo[rows], want) <= TOL["logits"]
    _check_route(ids, probs, lo, T, cfg.K, cfg.score, None if bias is None else r["bias"].numpy())


@pytest.mark.parametrize("E,K,H,wdt,T", [(32, 4, 576, torch.bfloat16, 77), (10, 3, 640, torch.float32, 300),
                                         (5, 5, 64, torch.bfloat16, 33)])
def test_route_small_router_from_x(E, K, H, wdt, T):
    """Small routers from bf16 rows (one workgroup per 32 tokens sums the H
    split across its wavefronts): ragged token tail, H that does not split
    evenly over the wavefronts, K = E, bf16 and fp32 router weights, bias and mask."""
    g = torch.Generator().manual_seed(E * 1000 + H)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    w = (torch.randn((H, E), generator=g) * 0.05).to(wdt)
    bias = torch.randn(E, generator=g) * 0.1
    mask = (torch.arange(T) % 7 == 3).to(torch.uint8)
    say("route small router", E, K, H, wdt, T)
    ids, probs, lo, err = _route_gpu(T, E, K, D.SOFTMAX, x=x.to(DEV), w_router=w.to(DEV), bias=bias.to(DEV),
                                     mask=mask.to(DEV))
    assert err == 0
    want = O.router_logits(to_numpy_f64(x), to_numpy_f64(w))
    assert rel_inf(lo, want) <= TOL["logits"]
    _check_route(ids, probs, lo, T, K, "softmax", bias.numpy(), mask.numpy())


@pytest.mark.parametrize("E", [4, 8, 10])
def test_route_small_router_uses_every_weight_term(E):
    """fp32 router weights reach the matrix cores as three bf16 terms
    (hi + mid + lo; term p of expert e is prepared row p * 10 + e).  With all
    of them summed, the projection is fp32-accurate: within 2e-6 of the
    float64 definition, where dropping the lo terms of some experts costs
    about 1e-5 (2^-17 of a weight)."""
    g = torch.Generator().manual_seed(77 + E)
    T, H, K = 64, 4096, 2
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    w = torch.randn((H, E), generator=g) * 0.05
    say("route small router weight terms", E)
    ids, probs, lo, err = _route_gpu(T, E, K, D.SOFTMAX, x=x.to(DEV), w_router=w.to(DEV))
    assert err == 0
    want = O.router_logits(to_numpy_f64(x), to_numpy_f64(w))
    assert rel_inf(lo, want) <= 2e-6


@pytest.mark.parametrize("E,K,H,T", [(160, 6, 640, 1000), (300, 8, 1152, 777), (256, 8, 128, 100),
                                     (4096, 64, 256, 300)])
def test_route_gemm_projection(E, K, H, T):
    """bf16 router weights with at least 128 experts: the projection runs as a
    dense matrix-core GEMM in pieces along H.  Ragged token tiles, expert counts
    that leave part of a 256-column tile (or a second one) empty, H that splits
    into uneven pieces or a single one, bias and mask."""
    g = torch.Generator().manual_seed(E * 1000 + H + T)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    w = (torch.randn((H, E), generator=g) * 0.05).to(torch.bfloat16)
    bias = torch.randn(E, generator=g) * 0.1
    mask = (torch.arange(T) % 9 == 4).to(torch.uint8)
    say("route gemm projection", E, K, H, T)
    ids, probs, lo, err = _route_gpu(T, E, K, D.SIGMOID, x=x.to(DEV), w_router=w.to(DEV), bias=bias.to(DEV),
                                     mask=mask.to(DEV))
    assert err == 0
    want = O.router_logits(to_numpy_f64(x), to_numpy_f64(w))
    assert rel_inf(lo, want) <= TOL["logits"]
    _check_route(ids, probs, lo, T, K, "sigmoid", bias.numpy(), mask.numpy())


@pytest.mark.parametrize("T", [2048, 8192])
def test_route_sparse_share_logits(T):
    cfg = get_config("sparse_share")
    say("route sparse share", T)
    r = make_router_inputs(cfg, T=T)
    ids, probs, lo, err = _route_gpu(T, cfg.E, cfg.K, D.SOFTMAX, logits=r["logits"].to(DEV), mask=r["mask"].to(DEV))
    assert err == 0
    np.testing.assert_array_equal(lo, r["logits"].numpy())
    _check_route(ids, probs, lo, T, cfg.K, "softmax", mask=r["mask"].numpy())
    # the literal i.i.d. N(0,1) logits too (route-only measurement shape)
    z = torch.randn((T, cfg.E), generator=torch.Generator().manual_seed(55))
    ids, probs, lo, err = _route_gpu(T, cfg.E, cfg.K, D.SOFTMAX, logits=z.to(DEV))
    _check_route(ids, probs, lo, T, cfg.K, "softmax")


@pytest.mark.parametrize("E,K", [(8, 1), (8, 8), (16, 5), (32, 32), (33, 3), (64, 64), (100, 36), (256, 8),
                                 (300, 36), (1024, 64), (1025, 2), (2304, 36), (4096, 64)])
@pytest.mark.parametrize("kind", ["normal", "ties", "equal", "signed_zero"])
def test_route_selection_edge_cases(E, K, kind):
    T = 300
    g = torch.Generator().manual_seed(E * 7 + K)
    if kind == "normal":
        z = torch.randn((T, E), generator=g)
    elif kind == "ties":
        z = torch.randint(0, 4, (T, E), generator=g).float() * 0.5
    elif kind == "equal":
        z = torch.full((T, E), 1.25)
    else:
        z = torch.randint(0, 2, (T, E), generator=g).float() * 0.0
        z[torch.rand((T, E), generator=g) < 0.5] *= -1.0
        z[:, ::5] = -1.0
    for score in (D.SOFTMAX, D.SIGMOID):
        ids, probs, lo, err = _route_gpu(T, E, K, score, logits=z.to(DEV))
        assert err == 0
        _check_route(ids, probs, lo, T, K, "softmax" if score == D.SOFTMAX else "sigmoid")


def test_route_nonfinite_sets_error_bit():
    z = torch.randn((64, 300))
    z[3, 7] = float("nan")
    _, _, _, err = _route_gpu(64, 300, 8, D.SOFTMAX, logits=z.to(DEV))
    assert err & D.DEVERR_NONFINITE
    z = torch.randn((64, 8))
    z[1, 2] = float("inf")
    _, _, _, err = _route_gpu(64, 8, 2, D.SOFTMAX, logits=z.to(DEV))
    assert err & D.DEVERR_NONFINITE


def test_route_bias_and_mask_small_and_large():
    for E, K in ((8, 2), (256, 8), (1025, 4), (2304, 36)):
        T = 200
        z = torch.randn((T, E), generator=torch.Generator().manual_seed(3))
        bias = torch.randn(E, generator=torch.Generator().manual_seed(4))
        mask = (torch.arange(T) % 3 == 0).to(torch.uint8)
        ids, probs, lo, err = _route_gpu(T, E, K, D.SIGMOID, logits=z.to(DEV), bias=bias.to(DEV), mask=mask.to(DEV))
        _check_route(ids, probs, lo, T, K, "sigmoid", bias.numpy(), mask.numpy())
        assert (ids[mask.numpy() == 1] == -1).all()


@pytest.mark.parametrize("counts,C", [([40, 0, 130, 1, 300], 128), ([0, 0], 64), ([1011, 1049, 983, 992], 4096)])
def test_mx_quantize_columns_grouped(counts, C):
    """Group-aware column-wise MX quantization: block offsets, codes and scales
    bit-exact against the oracle (each group blocked on its own, zero padding);
    blocks past the last group untouched."""
    rng = np.random.default_rng(sum(counts) + C)
    L = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    cap = int(offsets[-1]) + 20
    v = O.bf16_round(rng.standard_normal((cap, C)) * np.exp(rng.uniform(-6, 6, (cap, 1))))
    nbmax = D.moe_mx_columns_grouped_max_blocks(L, cap)
    pb = torch.full((L + 1,), -5, dtype=torch.int32, device=DEV)
    codes = torch.full((nbmax, C, 32), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((nbmax, C), 0xCD, dtype=torch.uint8, device=DEV)
    say("mx columns grouped", counts, C)
    D.moe_mx_quantize_columns_grouped(bf16_from_f64(v), torch.from_numpy(offsets).to(DEV), pb, codes, scales)
    torch.cuda.synchronize()
    opb, oc, os_ = O.mx_quantize_columns_grouped(v, offsets)
    np.testing.assert_array_equal(np_of(pb), opb)
    nb = int(opb[-1])
    np.testing.assert_array_equal(np_of(codes)[:nb], oc)
    np.testing.assert_array_equal(np_of(scales)[:nb], os_)
    assert (np_of(codes)[nb:] == 0xAB).all() and (np_of(scales)[nb:] == 0xCD).all()
