"""GPU parity of the grouped MLP's data gradient (moe_grouped_mlp_backward_data,
bf16 and MXFP8): d_x_perm against the oracle's chain rule with the same
rounding points (h and d_h stored as bf16; MX operands along each
contraction), within the bf16 / MXFP8 tolerance; the backward's W1^T and W2^T
panels exactly (bf16 values, or E4M3 codes and E8M0 scales); rows past N
untouched."""
import numpy as np
import pytest
import torch

import dropless_mixture_experts_radix_amd as D
from oracle import moe_oracle as O
from tests.gpu_util import DEV, TOL, bf16_from_f64, rel_inf, say, to_f64
from tests.test_gpu_mlp import MIXTRAL_COUNTS, _unblock, _weights

pytestmark = pytest.mark.gpu


def _mx_panels(codes, scales, L, P, K, e):
    """Codes [P][K] and scales [P][K/32] of expert e from MX panels (codes
    [L][P/256][K/64][256][64], scales [L][P/256][ceil(K/512)][256][16])."""
    NP, NG = P // 256, (K + 511) // 512
    c = codes.cpu().numpy().reshape(L, NP, K // 64, 256, 64)[e].transpose(0, 2, 1, 3).reshape(P, K)
    s = scales.cpu().numpy().reshape(L, NP, NG, 256, 16)[e].transpose(0, 2, 1, 3).reshape(P, NG * 16)
    return c, s[:, :K // 32]


def _run(counts, H, F, seed, sample=None, dt="bf16"):
    rng = np.random.default_rng(seed)
    L = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    cap = N + 24
    W1, W2 = _weights(rng, L, H, F, "bf16")
    x = O.bf16_round(rng.standard_normal((cap, H)))
    dy = O.bf16_round(rng.standard_normal((cap, H)))
    w1 = torch.stack([bf16_from_f64(w) for w in W1])
    w2 = torch.stack([bf16_from_f64(w) for w in W2])
    code = D.BF16 if dt == "bf16" else D.MXFP8
    nb = lambda which: torch.empty(max(D.moe_prepared_weight_bytes(L, H, F, code, which), 1), dtype=torch.uint8,
                                   device=DEV)
    w1p, w2p, w1t, w2t = nb(1), nb(2), nb(5), nb(6)
    if dt == "bf16":
        D.moe_prepare_weights(w1, w2, D.BF16, w1p.view(torch.bfloat16), w2p.view(torch.bfloat16))
        D.moe_prepare_weights_backward(w1, w2, w1t, w2t)
        sc = {}
    else:
        w1s, w2s, w1ts, w2ts = nb(3), nb(4), nb(7), nb(8)
        D.moe_prepare_weights(w1, w2, D.MXFP8, w1p, w2p, w1s, w2s)
        D.moe_prepare_weights_backward(w1, w2, w1t, w2t, w1ts, w2ts, dtype=D.MXFP8)
        sc = dict(w1p_scales=w1s, w1t_scales=w1ts, w2t_scales=w2ts)
    ws = torch.empty(D.moe_grouped_mlp_backward_workspace_bytes(cap, H, F, code), dtype=torch.uint8, device=DEV)
    dx = torch.full((cap, H), 5.0, dtype=torch.bfloat16, device=DEV)
    say("mlp backward data", dt, "L", L, "H", H, "F", F, "N", N)
    D.moe_grouped_mlp_backward_data(bf16_from_f64(x), torch.from_numpy(offsets).to(DEV), w1p, w1t, w2t,
                                    bf16_from_f64(dy), dx, ws, H, F, dtype=code, **sc)
    torch.cuda.synchronize()
    # the backward panels of the last expert, decoded
    e = L - 1
    pw1 = ((H + 255) // 256) * 256
    pw2 = ((F + 255) // 256) * 256
    if dt == "bf16":
        t1 = _unblock(w1t.view(torch.bfloat16).view(L, pw1, 2 * F)[e])
        t2 = _unblock(w2t.view(torch.bfloat16).view(L, pw2, H)[e])
        np.testing.assert_array_equal(t1[:H], W1[e])            # row h of W1^T panels = W1[e][h, :]
        np.testing.assert_array_equal(t2[:F], W2[e])            # row f of W2^T panels = W2[e][f, :]
        assert (t1[H:] == 0).all() and (t2[F:] == 0).all()
    else:  # MX panels: row h of W1^T = W1[e][h, :] quantized along 2F, row f of W2^T = W2[e][f, :] along H
        for (cd, scl, P, K, W) in ((w1t, w1ts, pw1, 2 * F, W1[e]), (w2t, w2ts, pw2, H, W2[e])):
            c, s = _mx_panels(cd, scl, L, P, K, e)
            wc, wsc = O.mx_quantize_rows(W)
            np.testing.assert_array_equal(c[:W.shape[0]], wc)
            np.testing.assert_array_equal(s[:W.shape[0]], wsc.reshape(W.shape[0], -1))
            assert (c[W.shape[0]:] == 0).all()
    got = to_f64(dx)
    assert (got[N:] == 5.0).all()
    if N == 0:
        return
    # the oracle on all rows, or on a sample of rows per expert (rows are independent)
    rows = np.arange(N) if sample is None else np.concatenate(
        [np.arange(offsets[k], offsets[k + 1])[:sample] for k in range(L)])
    sub_counts = [int(((rows >= offsets[k]) & (rows < offsets[k + 1])).sum()) for k in range(L)]
    sub_off = np.concatenate([[0], np.cumsum(sub_counts)])
    want = O.grouped_mlp_backward_data(x[rows], sub_off, W1, W2, dy[rows], dt)
    err = rel_inf(got[rows], want)
    say("  d_x rel err", err)
    assert err <= TOL[dt]


@pytest.mark.parametrize("counts,H,F", [
    ([0, 1, 255, 256, 257, 600, 0, 31], 256, 256),   # empty experts, ragged and tall tiles
    ([70, 300, 0, 5], 384, 128),                      # partial column tiles in all three GEMMs
    ([0, 0, 0], 128, 128),                            # no rows
    (MIXTRAL_COUNTS, 512, 512),                       # split-K pieces with tall tiles
])
def test_grouped_mlp_backward_data(counts, H, F):
    _run(counts, H, F, seed=sum(counts) + H + F)


def test_grouped_mlp_backward_data_mixtral_size():
    """The Mixtral-like shape (H = 4096, F = 14336, 8192 rows), checked on 48
    rows per expert."""
    _run(MIXTRAL_COUNTS, 4096, 14336, seed=7, sample=48)


@pytest.mark.parametrize("counts,H,F", [
    ([0, 1, 255, 256, 257, 600, 0, 31], 256, 256),   # empty experts, ragged and tall tiles
    ([70, 300, 0, 5], 512, 256),                      # H > 2F: partial split pieces
    ([0, 0, 0], 256, 256),                            # no rows
    (MIXTRAL_COUNTS, 512, 512),                       # split-K pieces with tall tiles
])
def test_grouped_mlp_backward_data_mxfp8(counts, H, F):
    _run(counts, H, F, seed=sum(counts) + 3 * H + F, dt="mxfp8")


def test_grouped_mlp_backward_data_mxfp8_mixtral_size():
    """MXFP8 at the Mixtral-like shape, checked on 48 rows per expert."""
    _run(MIXTRAL_COUNTS, 4096, 14336, seed=8, sample=48, dt="mxfp8")


def _run_wgrad(counts, H, F, seed, dt="bf16"):
    rng = np.random.default_rng(seed)
    L = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    cap = N + 24
    W1, W2 = _weights(rng, L, H, F, "bf16")
    x = O.bf16_round(rng.standard_normal((cap, H)))
    dy = O.bf16_round(rng.standard_normal((cap, H)))
    w1 = torch.stack([bf16_from_f64(w) for w in W1])
    w2 = torch.stack([bf16_from_f64(w) for w in W2])
    w1p = torch.empty(D.moe_prepared_weight_bytes(L, H, F, D.BF16, 1), dtype=torch.uint8, device=DEV)
    w2p = torch.empty(D.moe_prepared_weight_bytes(L, H, F, D.BF16, 2), dtype=torch.uint8, device=DEV)
    w1t = torch.empty(D.moe_prepared_weight_bytes(L, H, F, D.BF16, 5), dtype=torch.uint8, device=DEV)
    w2t = torch.empty(D.moe_prepared_weight_bytes(L, H, F, D.BF16, 6), dtype=torch.uint8, device=DEV)
    D.moe_prepare_weights(w1, w2, D.BF16, w1p.view(torch.bfloat16), w2p.view(torch.bfloat16))
    D.moe_prepare_weights_backward(w1, w2, w1t, w2t)
    ws = torch.empty(D.moe_grouped_mlp_backward_workspace_bytes(cap, H, F, D.BF16), dtype=torch.uint8, device=DEV)
    code = D.BF16 if dt == "bf16" else D.MXFP8
    wws = torch.empty(D.moe_grouped_mlp_backward_weights_workspace_bytes(L, cap, H, F, code), dtype=torch.uint8,
                      device=DEV)
    dx = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    dW1 = torch.full((L, H, 2 * F), 7.0, dtype=torch.float32, device=DEV)
    dW2 = torch.full((L, F, H), 7.0, dtype=torch.float32, device=DEV)
    off_d = torch.from_numpy(offsets).to(DEV)
    xd, dyd = bf16_from_f64(x), bf16_from_f64(dy)
    say("mlp backward weights L", L, "H", H, "F", F, "N", N)
    D.moe_grouped_mlp_backward_data(xd, off_d, w1p, w1t, w2t, dyd, dx, ws, H, F)
    D.moe_grouped_mlp_backward_weights(xd, off_d, dyd, ws, dW1, dW2, wws, H, F, dtype=code)
    torch.cuda.synchronize()
    want1, want2 = O.grouped_mlp_backward_weights(x[:N], offsets, W1, W2, dy[:N], dt)
    got1, got2 = dW1.cpu().numpy().astype(np.float64), dW2.cpu().numpy().astype(np.float64)
    for e, c in enumerate(counts):
        if c == 0:
            assert (got1[e] == 0).all() and (got2[e] == 0).all()
    e1, e2 = rel_inf(got1, want1), rel_inf(got2, want2)
    say("  dW1 rel err", e1, "dW2 rel err", e2)
    # bf16 intermediates (a, d_h) may differ by one rounding from the oracle's
    assert e1 <= TOL[dt] and e2 <= TOL[dt]


@pytest.mark.parametrize("counts,H,F", [
    ([0, 1, 31, 128, 129, 300, 0], 256, 256),   # empty experts, rows not a multiple of 32 or 128
    ([70, 300, 0, 5], 384, 128),                 # partial I and J tiles
    (MIXTRAL_COUNTS, 512, 512),
])
def test_grouped_mlp_backward_weights(counts, H, F):
    _run_wgrad(counts, H, F, seed=sum(counts) + 3 * H + F)


@pytest.mark.parametrize("counts,H,F", [
    ([0, 1, 31, 128, 129, 300, 0], 256, 256),   # empty experts, rows padded to 256 per expert
    ([70, 300, 0, 5], 384, 128),                 # partial I and J tiles
    (MIXTRAL_COUNTS, 512, 512),                  # several 512-row scale groups per expert
])
def test_grouped_mlp_backward_weights_mxfp8(counts, H, F):
    """MXFP8 weight gradient: group-aware column-wise MX operands, MX matrix-core
    GEMMs; against the oracle's MXFP8 path within the MX tolerance."""
    _run_wgrad(counts, H, F, seed=sum(counts) + 5 * H + F, dt="mxfp8")
