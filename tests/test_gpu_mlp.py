"""GPU parity of the grouped SwiGLU MLP (fp32 1e-5, bf16 2e-2, MXFP8 3e-2 of
the oracle's largest magnitude), the prepared weight layouts (bit-exact,
including the MX codes and scales of the weights), the MX codes and scales of
the activations bit-exact against the quantizer's definition on the GPU's own
bf16 `a` (moe_grouped_mlp_with_act), ragged groups spanning several tiles,
empty experts, partial column tiles and untouched rows."""
import numpy as np
import pytest
import torch

import dropless_mixture_experts_radix_amd as D
from oracle import moe_oracle as O
from tests.gpu_util import DEV, TOL, bf16_from_f64, np_of, rel_inf, say, to_f64

pytestmark = pytest.mark.gpu

DT = {"f32": D.F32, "bf16": D.BF16, "mxfp8": D.MXFP8, "mxfp4": D.MXFP4}


def _interleave_rows(F):
    p = np.arange(2 * F)
    return (p // 64) * 32 + p % 32 + np.where((p // 32) % 2 == 1, F, 0)


def _unblock(wp):
    """bf16 prepared weights of one expert, k-blocked panels [rows/256][Kd/32][256][32],
    back to rows x Kd (float64)."""
    rows, kd = wp.shape
    t = wp.reshape(rows // 256, kd // 32, 256, 32).permute(0, 2, 1, 3)   # panel, r, kt, e
    return to_f64(t.reshape(rows, kd))


def _unblock_mx(wp, ws, fp4=False):
    """MX prepared weights of one expert, k-blocked panels: codes
    [rows/256][Kd/64 bytes][256][64] (MXFP4: 64 bytes = 128 codes) and scales
    [rows/256][ceil(Kd/512)][256][16], back to row-major code bytes [rows][Kd
    or Kd/2] and scales [rows][Kd/32] (numpy uint8)."""
    rows, kb = wp.shape  # code bytes per row
    kd = kb * 2 if fp4 else kb
    ng = (kd + 511) // 512
    c = np_of(wp).reshape(rows // 256, kb // 64, 256, 64).transpose(0, 2, 1, 3).reshape(rows, kb)
    s = np_of(ws).reshape(rows // 256, ng, 256, 16).transpose(0, 2, 1, 3).reshape(rows, ng * 16)[:, : kd // 32]
    return c, s


MIXTRAL_COUNTS = [1011, 1049, 983, 992, 1052, 1081, 977, 1047]


def _weights(rng, L, H, F, dt, scale=0.05):
    W1 = [rng.standard_normal((H, 2 * F)) * scale for _ in range(L)]
    W2 = [rng.standard_normal((F, H)) * scale for _ in range(L)]
    if dt == "f32":
        W1 = [w.astype(np.float32).astype(np.float64) for w in W1]
        W2 = [w.astype(np.float32).astype(np.float64) for w in W2]
    else:
        W1 = [O.bf16_round(w) for w in W1]
        W2 = [O.bf16_round(w) for w in W2]
    return W1, W2


def _dev(v, dt):
    if dt == "f32":
        return torch.from_numpy(np.asarray(v, np.float32)).to(DEV)
    return bf16_from_f64(np.asarray(v))


def _run_mlp(counts, H, F, dt, seed=0, xscale=1.0, check_layout=True):
    rng = np.random.default_rng(seed)
    L = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    cap = N + 40
    W1, W2 = _weights(rng, L, H, F, dt)
    x64 = rng.standard_normal((cap, H)) * xscale
    x64 = x64.astype(np.float32).astype(np.float64) if dt == "f32" else O.bf16_round(x64)
    code = DT[dt]
    w1 = torch.stack([_dev(w, dt) for w in W1])
    w2 = torch.stack([_dev(w, dt) for w in W2])
    mx = dt in ("mxfp8", "mxfp4")
    wdt = {"f32": torch.float32, "bf16": torch.bfloat16, "mxfp8": torch.uint8, "mxfp4": torch.uint8}[dt]
    pad = (lambda n: (n + 255) // 256 * 256) if dt != "f32" else (lambda n: n)
    cw = (lambda n: n // 2) if dt == "mxfp4" else (lambda n: n)
    w1p = torch.empty((L, pad(2 * F), cw(H)), dtype=wdt, device=DEV)
    w2p = torch.empty((L, pad(H), cw(F)), dtype=wdt, device=DEV)
    w1s = w2s = None
    if mx:
        w1s = torch.empty((L, pad(2 * F), (H + 511) // 512 * 16), dtype=torch.uint8, device=DEV)
        w2s = torch.empty((L, pad(H), (F + 511) // 512 * 16), dtype=torch.uint8, device=DEV)
    D.moe_prepare_weights(w1, w2, code, w1p, w2p, w1s, w2s)
    perm = _interleave_rows(F)
    if check_layout:
        e = L - 1
        if mx:
            quant = O.mx_quantize_rows if dt == "mxfp8" else (lambda m: (lambda c, s: (O.pack_fp4(c), s))(
                *O.mx4_quantize_rows(m)))
            c1, s1 = quant(W1[e].T[perm])
            c2, s2 = quant(W2[e].T)
            w1c, w1sc = _unblock_mx(w1p[e], w1s[e], dt == "mxfp4")
            w2c, w2sc = _unblock_mx(w2p[e], w2s[e], dt == "mxfp4")
            np.testing.assert_array_equal(w1c[: 2 * F], c1)
            np.testing.assert_array_equal(w1sc[: 2 * F], s1)
            np.testing.assert_array_equal(w2c[:H], c2)
            np.testing.assert_array_equal(w2sc[:H], s2)
            assert (w1c[2 * F:] == 0).all() and (w1sc[2 * F:] == 0).all()
            assert (w2c[H:] == 0).all() and (w2sc[H:] == 0).all()
        elif dt == "bf16":
            np.testing.assert_array_equal(_unblock(w1p[e])[: 2 * F], W1[e].T[perm])
            np.testing.assert_array_equal(_unblock(w2p[e])[:H], W2[e].T)
            assert (_unblock(w1p[e])[2 * F:] == 0).all() and (_unblock(w2p[e])[H:] == 0).all()
        else:
            np.testing.assert_array_equal(to_f64(w1p[e]), W1[e].T[perm])
            np.testing.assert_array_equal(to_f64(w2p[e]), W2[e].T)
    xd = _dev(x64, "f32" if dt == "f32" else "bf16")
    xs = None
    if dt == "mxfp8":
        xq = torch.empty((cap, H), dtype=torch.uint8, device=DEV)
        xs = torch.empty((cap, H // 32), dtype=torch.uint8, device=DEV)
        D.moe_mx_quantize(xd, xq, xs)
        xd = xq
    elif dt == "mxfp4":  # quantized rows from the oracle (the permute's own are pinned on their own)
        c, s_ = O.mx4_quantize_rows(x64)
        xd = torch.from_numpy(O.pack_fp4(c)).to(DEV)
        xs = torch.from_numpy(s_).to(DEV)
    ydt = torch.float32 if dt == "f32" else torch.bfloat16
    y = torch.full((cap, H), 5.0, dtype=ydt, device=DEV)
    ws = torch.empty(D.moe_grouped_mlp_workspace_bytes(cap, F, code), dtype=torch.uint8, device=DEV)
    off_d = torch.from_numpy(offsets).to(DEV)
    say("mlp", dt, "L", L, "H", H, "F", F, "N", N)
    act = None
    if mx:  # the epilogue's bf16 `a` as well (test hook), rows past N keep the sentinel
        act = torch.full((cap, F), 3.0, dtype=torch.bfloat16, device=DEV)
        D.moe_grouped_mlp_with_act(xd, off_d, w1p, w2p, y, ws, code, H, F, act, x_perm_scales=xs, w1p_scales=w1s,
                                   w2p_scales=w2s)
    else:
        D.moe_grouped_mlp(xd, off_d, w1p, w2p, y, ws, code, H, F, x_perm_scales=xs, w1p_scales=w1s,
                          w2p_scales=w2s)
    torch.cuda.synchronize()
    if mx:
        a_gpu = to_f64(act)
        assert (a_gpu[N:] == 3.0).all()
        a_gpu = a_gpu[:N]
    want_y, want_a = O.grouped_mlp(x64[:N], offsets, W1, W2, dt)
    got_y = to_f64(y)
    assert (got_y[N:] == 5.0).all()
    if N:
        say("  y rel err", rel_inf(got_y[:N], want_y))
        assert rel_inf(got_y[:N], want_y) <= TOL[dt], rel_inf(got_y[:N], want_y)
        if dt == "f32":
            a = ws[: cap * F * 4].view(torch.float32).view(cap, F)
            assert rel_inf(to_f64(a)[:N], want_a) <= TOL[dt]
        elif dt == "bf16":  # k-blocked activations [F/32][cap][32]
            a = ws[: cap * F * 2].view(torch.bfloat16).view(F // 32, cap, 32).permute(1, 0, 2).reshape(cap, F)
            assert rel_inf(to_f64(a)[:N], want_a) <= TOL[dt]
        elif dt == "mxfp4":
            cb = F // 2
            codes = O.unpack_fp4(np_of(ws[: cap * cb].view(cap, cb))[:N])
            off = (cap * cb + 255) // 256 * 256
            sc = np_of(ws[off: off + cap * (F // 32)].view(cap, F // 32))[:N]
            a_dq = O.mx4_dequantize_rows(codes, sc)
            # every element within half an E2M1 step (a quarter of its magnitude,
            # a quarter of its block scale below 2) of the oracle's bf16 `a`, or
            # clamped at 6 * 2^E, plus 1e-3 of the largest |a| for the fp32
            # accumulation inside the matrix cores
            scl = np.ldexp(1.0, sc.astype(np.int64) - 127).repeat(32, axis=1)
            bound = (np.maximum(np.abs(want_a) / 4, scl / 4) * (1 + 2.0 ** -7) + 1e-3 * np.abs(want_a).max() +
                     np.maximum(0.0, np.abs(want_a) * (1 + 2.0 ** -7) - 6 * scl))
            bad = np.argwhere(np.abs(a_dq - want_a) > bound)
            assert bad.size == 0, (len(bad), [(int(r), int(c), float(a_dq[r, c]), float(want_a[r, c]))
                                              for r, c in bad[:8]])
            # bit-exact: the codes and scales are the MX quantizer's definition
            # applied to the GPU's own bf16 `a`, which is within the bf16
            # tolerance of the oracle's
            assert rel_inf(a_gpu, want_a) <= TOL["bf16"]
            oc, os_ = O.mx4_quantize_rows(a_gpu)
            np.testing.assert_array_equal(codes, oc)
            np.testing.assert_array_equal(sc, os_)
            mags = O.e2m1_decode(codes & 7).reshape(N, F // 32, 32).max(axis=2)
            nz = mags > 0
            big = O.mx4_dequantize_rows(codes, sc).reshape(N, F // 32, 32)
            assert ((mags[nz] >= 4) | (np.abs(big).max(axis=2)[nz] < 2.0 ** -124)).all()
        else:
            codes = np_of(ws[: cap * F].view(cap, F))[:N]
            off = (cap * F + 255) // 256 * 256
            sc = np_of(ws[off: off + cap * (F // 32)].view(cap, F // 32))[:N]
            a_dq = O.mx_dequantize_rows(codes, sc)
            # every element within half an E4M3 step of the oracle's bf16 `a`, or clamped
            # at 448 * 2^E where the MX conversion saturates, plus an absolute slack of
            # 1e-3 of the largest |a| for the fp32 accumulation inside the matrix cores
            scl = np.ldexp(1.0, sc.astype(np.int64) - 127).repeat(32, axis=1)
            bound = (np.abs(want_a) * (2.0 ** -4 + 2.0 ** -7) + 1e-3 * np.abs(want_a).max() +
                     np.maximum(0.0, np.abs(want_a) * (1 + 2.0 ** -7) - 448 * scl))
            bad = np.argwhere(np.abs(a_dq - want_a) > bound)
            assert bad.size == 0, (len(bad), [(int(r), int(c), float(a_dq[r, c]), float(want_a[r, c]))
                                              for r, c in bad[:8]])
            # bit-exact: the codes and scales are the MX quantizer's definition
            # applied to the GPU's own bf16 `a`, which is within the bf16
            # tolerance of the oracle's
            assert rel_inf(a_gpu, want_a) <= TOL["bf16"]
            oc, os_ = O.mx_quantize_rows(a_gpu)
            np.testing.assert_array_equal(codes, oc)
            np.testing.assert_array_equal(sc, os_)
            # scale rule: every non-zero block's largest code magnitude lies in [256, 448]
            mags = O.e4m3_decode(codes & 0x7F).reshape(N, F // 32, 32).max(axis=2)
            nz = mags > 0
            big = O.mx_dequantize_rows(codes, sc).reshape(N, F // 32, 32)
            assert ((mags[nz] >= 256) | (np.abs(big).max(axis=2)[nz] < 2.0 ** -118)).all()
    return got_y, want_y


@pytest.mark.parametrize("counts,H,F", [([100, 0, 37, 256], 64, 128), ([3, 1, 0, 4], 32, 32),
                                        ([300, 65, 0, 1, 64], 96, 64)])
def test_grouped_mlp_f32(counts, H, F):
    _run_mlp(counts, H, F, "f32", seed=sum(counts))


@pytest.mark.parametrize("counts,H,F", [
    ([0, 1, 255, 256, 257, 600, 0, 31], 256, 512),
    ([1000, 24, 0, 513], 1024, 1536),
    ([70, 300, 0, 5], 384, 128),          # partial column tiles in both GEMMs
    ([0, 0, 0, 0], 256, 256),             # no rows at all
    ([2048], 512, 512),
    # 8192 routed rows over 8 experts (33 row tiles, three of them tall) on a
    # 256-CU grid: the 66 tiles of a partial round are split along k into 3
    # uneven pieces (first GEMM: k = 3584, 28 groups of 4 steps; second GEMM:
    # k = 4096, 32 groups), tall tiles among them
    (MIXTRAL_COUNTS, 3584, 256),
    (MIXTRAL_COUNTS, 512, 4096),
    # tall tiles (an expert takes ceil(m / 320) tiles of up to 256 + 64 rows):
    # 257-321 rows in one tile (the extra rows of one or both wavefront
    # groups), 544 as 288 + 256, a lone 31
    ([257, 272, 288, 289, 544, 0, 31], 512, 512),
    # the extra rows spread over an expert's first tiles: 1124 = 320 + 292 +
    # 256 + 256, 1201 = 320 + 320 + 305 + 256, 1088 = 320 + 3 x 256, and 321
    # as 256 + 65
    ([1124, 320, 321, 1201, 0, 7, 1088], 512, 512),
    # tall tiles in whole rounds of the first GEMM (256 tiles on 256 CUs)
    ([1054, 994, 1030, 1018, 1040, 1008, 1024, 1024], 512, 1024),
])
def test_grouped_mlp_bf16(counts, H, F):
    _run_mlp(counts, H, F, "bf16", seed=sum(counts) + H)


@pytest.mark.parametrize("counts,H,F", [
    ([0, 1, 255, 256, 257, 600, 0, 31], 256, 512),
    ([900, 24, 0, 513], 1024, 1536),
    ([70, 300, 0, 5], 768, 256),          # partial column tiles in both GEMMs
    ([0, 0, 0, 0], 256, 256),             # no rows at all
    # the 66 tiles of a partial round (tall ones among them) split along k
    # into 2 pieces (first GEMM: k = 4096; second GEMM: k = 4096)
    (MIXTRAL_COUNTS, 4096, 256),
    (MIXTRAL_COUNTS, 512, 4096),
    # tall tiles (an expert takes ceil(m / 288) tiles of up to 256 + 32 rows):
    # 257-288 rows in one tile, 289 as 256 + 33, 544 as 288 + 256, a lone 31
    ([257, 272, 288, 289, 544, 0, 31], 512, 512),
    ([1054, 994, 1030, 1018, 1040, 1008, 1024, 1024], 512, 1024),
])
def test_grouped_mlp_mxfp8(counts, H, F):
    _run_mlp(counts, H, F, "mxfp8", seed=sum(counts) + H)


@pytest.mark.parametrize("counts,H,F", [
    ([0, 1, 255, 256, 257, 600, 0, 31], 512, 512),
    ([900, 24, 0, 513], 1024, 1536),
    ([70, 300, 0, 5], 1536, 512),         # partial column tiles in both GEMMs
    ([0, 0, 0, 0], 512, 512),             # no rows at all
    # 4028 rows (17 row tiles): the 68 tiles of the first GEMM (k = 8192, 16
    # groups of 4 E2M1 stages) and the 34 of the second (k = 8192) are split
    # along k into 2 pieces
    ([1000, 1011, 977, 1040], 8192, 512),
    ([1000, 1011, 977, 1040], 512, 8192),
    # remainders of 1 to 33 rows after full tiles (tall tiles in the bf16 and
    # E4M3 kernels; the E2M1 kernel keeps them in tiles of their own)
    ([257, 272, 288, 289, 544, 0, 31], 512, 512),
    ([1054, 994, 1030, 1018, 1040, 1008, 1024, 1024], 512, 1024),
])
def test_grouped_mlp_mxfp4(counts, H, F):
    _run_mlp(counts, H, F, "mxfp4", seed=sum(counts) + H + 1)
