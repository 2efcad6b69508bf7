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
from tests.gpu_util import DEV, TOL, bf16_from_f64, np_of, rel_inf, say, to_f64
from tests.test_gpu_mlp import MIXTRAL_COUNTS, _unblock, _weights

pytestmark = pytest.mark.gpu


def _mx_panels(codes, scales, L, P, K, e):
    """Codes [P][K] and scales [P][K/32] of expert e from MX panels (codes
    [L][P/256][K/64][256][64], scales [L][P/256][ceil(K/512)][256][16])."""
    NP, NG = P // 256, (K + 511) // 512
    c = codes.cpu().numpy().reshape(L, NP, K // 64, 256, 64)[e].transpose(0, 2, 1, 3).reshape(P, K)
    s = scales.cpu().numpy().reshape(L, NP, NG, 256, 16)[e].transpose(0, 2, 1, 3).reshape(P, NG * 16)
    return c, s[:, :K // 32]


def _run(counts, H, F, seed, sample=None, dt="bf16", sample_experts=None):
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
        [np.arange(offsets[k], offsets[k + 1])[:sample] for k in (range(L) if sample_experts is None
                                                                   else sample_experts)])
    sub_counts = [int(((rows >= offsets[k]) & (rows < offsets[k + 1])).sum()) for k in range(L)]
    sub_off = np.concatenate([[0], np.cumsum(sub_counts)])
    want = O.grouped_mlp_backward_data(x[rows], sub_off, W1, W2, dy[rows], dt)
    err = rel_inf(got[rows], want)
    say("  d_x rel err", err)
    assert err <= TOL[dt]
    if dt == "mxfp8" and sample is None:  # (at the full size the oracle's MX pass over the weights takes minutes)
        _check_dh_mx(ws, cap, H, F, L, offsets, rows, x, dy, W1, W2)


def _check_dh_mx(ws, cap, H, F, L, offsets, rows, x, dy, W1, W2):
    """The MXFP8 data gradient's d_h (bf16, k-blocked [2F/32][capacity][32],
    gates then ups) and its row-wise MX codes and scales along 2F, as the
    workspace holds them: codes and scales bit-exact against the quantizer's
    definition applied to the GPU's own d_h; d_h itself within the bf16
    tolerance of the oracle's (its MX contractions, bf16 rounding points)."""
    z = D.moe_query_sizes(T=cap, H=H, E=L, K=1, F=F, dtype=D.MXFP8)  # capacity = cap
    assert z["capacity"] == cap
    o = z["bwd_dh_offset"]
    blk = ws[o: o + cap * 2 * F * 2].view(torch.bfloat16).view(2 * F // 32, cap, 32)
    dh = to_f64(blk.permute(1, 0, 2).reshape(cap, 2 * F)[rows])
    oc, osc = z["bwd_dh_codes_offset"], z["bwd_dh_scales_offset"]
    codes = np_of(ws[oc: oc + cap * 2 * F].view(cap, 2 * F))[rows]
    scales = np_of(ws[osc: osc + cap * (2 * F // 32)].view(cap, 2 * F // 32))[rows]
    wc, wsc = O.mx_quantize_rows(dh)
    np.testing.assert_array_equal(codes, wc)
    np.testing.assert_array_equal(scales, wsc.reshape(len(rows), -1))
    want = np.zeros_like(dh)
    for e in range(L):
        sel = (rows >= offsets[e]) & (rows < offsets[e + 1])
        if sel.any():
            want[sel] = O.mlp_backward_intermediates(x[rows[sel]], dy[rows[sel]], W1[e], W2[e], "mxfp8")[2]
    err = rel_inf(dh, want)
    say("  d_h rel err", err, "(MX codes and scales of d_h bit-exact)")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("counts,H,F", [
    ([0, 1, 255, 256, 257, 600, 0, 31], 256, 256),   # empty experts, ragged and tall tiles
    ([70, 300, 0, 5], 384, 128),                      # partial column tiles in all three GEMMs
    ([0, 0, 0], 128, 128),                            # no rows
    (MIXTRAL_COUNTS, 512, 512),                       # split-K pieces with tall tiles
    ([1124, 320, 321, 1201, 0, 7], 256, 256),         # extra rows over an expert's first tiles
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
    """MXFP8 at the Mixtral-like shape, checked on 48 rows of the first and the
    last expert (the oracle's MX pass over one expert's full weights takes
    about a minute of CPU time)."""
    _run(MIXTRAL_COUNTS, 4096, 14336, seed=8, sample=48, dt="mxfp8", sample_experts=(0, 7))


def _run_wgrad(counts, H, F, seed, dt="bf16", data_dt="bf16"):
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
    dcode = D.BF16 if data_dt == "bf16" else D.MXFP8
    nb = lambda which: torch.empty(max(D.moe_prepared_weight_bytes(L, H, F, dcode, which), 1), dtype=torch.uint8,
                                   device=DEV)
    w1p, w2p, w1t, w2t = nb(1), nb(2), nb(5), nb(6)
    sc = {}
    if data_dt == "bf16":
        D.moe_prepare_weights(w1, w2, D.BF16, w1p.view(torch.bfloat16), w2p.view(torch.bfloat16))
        D.moe_prepare_weights_backward(w1, w2, w1t, w2t)
    else:  # the weight gradient follows an MXFP8 data pass (its h and d_h)
        w1s, w2s, w1ts, w2ts = nb(3), nb(4), nb(7), nb(8)
        D.moe_prepare_weights(w1, w2, D.MXFP8, w1p, w2p, w1s, w2s)
        D.moe_prepare_weights_backward(w1, w2, w1t, w2t, w1ts, w2ts, dtype=D.MXFP8)
        sc = dict(dtype=D.MXFP8, w1p_scales=w1s, w1t_scales=w1ts, w2t_scales=w2ts)
    ws = torch.empty(D.moe_grouped_mlp_backward_workspace_bytes(cap, H, F, dcode), dtype=torch.uint8, device=DEV)
    code = D.BF16 if dt == "bf16" else D.MXFP8
    wws = torch.empty(D.moe_grouped_mlp_backward_weights_workspace_bytes(L, cap, H, F, code), dtype=torch.uint8,
                      device=DEV)
    dx = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    dW1 = torch.full((L, H, 2 * F), 7.0, dtype=torch.float32, device=DEV)
    dW2 = torch.full((L, F, H), 7.0, dtype=torch.float32, device=DEV)
    off_d = torch.from_numpy(offsets).to(DEV)
    xd, dyd = bf16_from_f64(x), bf16_from_f64(dy)
    say("mlp backward weights", dt, "after a", data_dt, "data pass: L", L, "H", H, "F", F, "N", N)
    D.moe_grouped_mlp_backward_data(xd, off_d, w1p, w1t, w2t, dyd, dx, ws, H, F, **sc)
    D.moe_grouped_mlp_backward_weights(xd, off_d, dyd, ws, dW1, dW2, wws, H, F, dtype=code)
    torch.cuda.synchronize()
    want1, want2 = O.grouped_mlp_backward_weights(x[:N], offsets, W1, W2, dy[:N], dt, data_dtype=data_dt)
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


@pytest.mark.parametrize("counts,H,F", [
    ([0, 1, 31, 128, 129, 300, 0], 256, 256),   # empty experts, rows padded to 256 per expert
    (MIXTRAL_COUNTS, 512, 512),                  # split-K pieces in the data pass, several scale groups
])
def test_grouped_mlp_backward_mxfp8_data_then_weights(counts, H, F):
    """The MXFP8 training chain: the MXFP8 data gradient, then the MXFP8 weight
    gradient on the h and d_h that pass left in its workspace, against the
    oracle's composition (weight_gradient_operands of an MXFP8 data pass, then
    the group-aware column-wise MX contraction)."""
    _run_wgrad(counts, H, F, seed=sum(counts) + 7 * H + F, dt="mxfp8", data_dt="mxfp8")


def test_grouped_mlp_backward_mxfp8_operands_from_producers():
    """The MXFP8 data gradient given the row-wise MX operands of x_perm and d_y
    by their producers (the MXFP8 permute's codes of the token rows; the
    combine backward's MX output of d_y) instead of quantizing the bf16 rows
    itself: the same codes enter the same GEMMs, so d_x is bit-identical to
    the self-quantizing call, and the workspace's h and d_h too."""
    rng = np.random.default_rng(31)
    T, E, K, H, F = 700, 8, 2, 512, 512
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, probs = O.route_topk(logits, K, "softmax")
    x64 = O.bf16_round(rng.standard_normal((T, H)))
    cap = T * K
    ids_d = torch.from_numpy(ids).to(DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    r2s = torch.empty(cap, dtype=torch.int32, device=DEV)
    s2r = torch.empty((T, K), dtype=torch.int32, device=DEV)
    xb = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    xq = torch.empty((cap, H), dtype=torch.uint8, device=DEV)
    xqs = torch.empty((cap, H // 32), dtype=torch.uint8, device=DEV)
    ws = torch.zeros(D.moe_permute_workspace_bytes(T, K, E), dtype=torch.uint8, device=DEV)
    xd = bf16_from_f64(x64)
    D.moe_permute(xd, ids_d, E, 0, E, counts, offsets, xb, r2s, s2r, ws)                       # bf16 rows
    D.moe_permute(xd, ids_d, E, 0, E, counts, offsets, xq, r2s, s2r, ws, x_perm_scales=xqs,
                  out_dtype=D.MXFP8)                                                             # their MX codes
    y = bf16_from_f64(O.bf16_round(rng.standard_normal((cap, H))))
    dout = bf16_from_f64(O.bf16_round(rng.standard_normal((T, H))))
    dy = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    dyq = torch.empty((cap, H), dtype=torch.uint8, device=DEV)
    dyqs = torch.empty((cap, H // 32), dtype=torch.uint8, device=DEV)
    dp = torch.empty((T, K), dtype=torch.float32, device=DEV)
    D.moe_unpermute_combine_backward(dout, y, s2r, torch.from_numpy(probs).to(DEV), dy, dp, d_y_perm_q=dyq,
                                     d_y_perm_q_scales=dyqs)
    W1, W2 = _weights(rng, E, H, F, "bf16")
    w1 = torch.stack([bf16_from_f64(w) for w in W1])
    w2 = torch.stack([bf16_from_f64(w) for w in W2])
    nb = lambda which: torch.empty(D.moe_prepared_weight_bytes(E, H, F, D.MXFP8, which), dtype=torch.uint8,
                                   device=DEV)
    w1p, w2p, w1s, w2s, w1t, w2t, w1ts, w2ts = (nb(k) for k in (1, 2, 3, 4, 5, 6, 7, 8))
    D.moe_prepare_weights(w1, w2, D.MXFP8, w1p, w2p, w1s, w2s)
    D.moe_prepare_weights_backward(w1, w2, w1t, w2t, w1ts, w2ts, dtype=D.MXFP8)
    sc = dict(dtype=D.MXFP8, w1p_scales=w1s, w1t_scales=w1ts, w2t_scales=w2ts)
    wsz = D.moe_grouped_mlp_backward_workspace_bytes(cap, H, F, D.MXFP8)
    ws_a = torch.zeros(wsz, dtype=torch.uint8, device=DEV)
    ws_b = torch.zeros(wsz, dtype=torch.uint8, device=DEV)
    dx_a = torch.full((cap, H), 5.0, dtype=torch.bfloat16, device=DEV)
    dx_b = torch.full((cap, H), 5.0, dtype=torch.bfloat16, device=DEV)
    say("mxfp8 data gradient, operands from producers: T", T, "N", cap)
    D.moe_grouped_mlp_backward_data(xb, offsets, w1p, w1t, w2t, dy, dx_a, ws_a, H, F, **sc)
    D.moe_grouped_mlp_backward_data(None, offsets, w1p, w1t, w2t, None, dx_b, ws_b, H, F, x_perm_q=xq,
                                    x_perm_q_scales=xqs, d_y_perm_q=dyq, d_y_perm_q_scales=dyqs, **sc)
    torch.cuda.synchronize()
    N = int(offsets[-1].item())
    np.testing.assert_array_equal(to_f64(dx_b)[:N], to_f64(dx_a)[:N])
    assert (to_f64(dx_b)[N:] == 5.0).all()
    z = D.moe_query_sizes(T=cap, H=H, E=E, K=1, F=F, dtype=D.MXFP8)
    hd = z["bwd_dh_offset"] * 2  # h and d_h, k-blocked bf16, at the workspace's start
    np.testing.assert_array_equal(np_of(ws_b[:hd]), np_of(ws_a[:hd]))
