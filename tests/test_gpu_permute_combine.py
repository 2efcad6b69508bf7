"""GPU parity: count/scan/permute (bit-exact: counts, offsets, maps, rows, MX
codes and scales) and unpermute/combine (within tolerance), with the edge
cases: -1 routes, duplicate ids, non-local ids, bad ids, overflow, empty
input, untouched capacity rows, determinism."""
import numpy as np
import pytest
import torch

import dropless_mixture_experts_radix_amd as D
from oracle import moe_oracle as O
from tests.gpu_util import DEV, TOL, bf16_from_f64, np_of, rel_inf, say, to_f64

pytestmark = pytest.mark.gpu

SENT = -777


def _rand_ids(rng, T, K, E, p_inv=0.1, distinct=False):
    if distinct:
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :K]
    else:
        ids = rng.integers(0, E, size=(T, K))
    ids = ids.astype(np.int64)
    ids[rng.random((T, K)) < p_inv] = -1
    return ids.astype(np.int16)


def _state_bytes(T, K, L):
    """Bytes of the permute workspace's shared state (zero between calls)."""
    return D.moe_query_sizes(T=T, H=64, E=max(L, K), K=K, F=128, dtype=D.BF16, L=L)["permute_state_bytes"]


def _permute_gpu(x, ids, E, e0, L, capacity, out_dtype=None, ws=None, check_ws=True):
    T, H = x.shape
    K = ids.shape[1]
    counts = torch.full((L,), SENT, dtype=torch.int32, device=DEV)
    offsets = torch.full((L + 1,), SENT, dtype=torch.int32, device=DEV)
    mx = out_dtype in (D.MXFP8, D.MXFP4)
    width = H // 2 if out_dtype == D.MXFP4 else H
    x_perm = torch.full((max(capacity, 1), width), 0x5A if mx else 3.0,
                        dtype=torch.uint8 if mx else x.dtype, device=DEV)[:capacity]
    xs = torch.full((max(capacity, 1), H // 32), 0xC3, dtype=torch.uint8, device=DEV)[:capacity] if mx else None
    r2s = torch.full((capacity,), SENT, dtype=torch.int32, device=DEV)
    s2r = torch.full((T, K), SENT, dtype=torch.int32, device=DEV)
    state = _state_bytes(T, K, L) if T > 0 else 0
    if ws is None:
        # zero-filled state (the finished-tile counter and the tile counts); the
        # tile bases and slot rows after it poisoned (written before they are read)
        ws = torch.full((D.moe_permute_workspace_bytes(T, K, L),), 0xEE, dtype=torch.uint8, device=DEV)
        ws[:state] = 0
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    D.moe_permute(x, torch.from_numpy(ids).to(DEV), E, e0, L, counts, offsets, x_perm, r2s, s2r, ws,
                  x_perm_scales=xs, err=err, out_dtype=out_dtype)
    torch.cuda.synchronize()
    # the call leaves the state zero again
    if T > 0 and check_ws:
        assert int((ws[:state] != 0).sum().item()) == 0
    return dict(counts=np_of(counts), offsets=np_of(offsets), x_perm=x_perm, xs=xs, r2s=np_of(r2s),
                s2r=np_of(s2r), err=int(err.item()), ws=ws)


CASES = [(1000, 2, 8, 0, 8, 64), (257, 36, 2304, 0, 32, 512), (3000, 8, 256, 0, 256, 256), (100, 4, 16, 4, 8, 136),
         (1, 1, 1, 0, 1, 8), (5000, 1, 3, 1, 2, 64), (700, 64, 64, 0, 64, 32),
         # the sparse share's shape (293 tiles of 28 tokens, 36 routes each); 2048 local experts
         (8192, 36, 2304, 0, 32, 512), (4096, 8, 4096, 1024, 2048, 64),
         # the scan in several batches of tiles: 507 tiles of 79 tokens
         (40000, 36, 2304, 0, 32, 64),
         # tiles counted in several LDS chunks: 8 tiles of 20000 slots
         (20000, 8, 4096, 1024, 2048, 32)]


@pytest.mark.parametrize("T,K,E,e0,L,H", CASES)
def test_permute_bit_exact(T, K, E, e0, L, H):
    rng = np.random.default_rng(T + K + E)
    ids = _rand_ids(rng, T, K, E)
    x64 = O.bf16_round(rng.standard_normal((T, H)))
    x = bf16_from_f64(x64)
    ref = O.count_and_permute(ids, e0, L, x64, E_global=E)
    N = int(ref["offsets"][-1])
    cap = T * K
    say("permute", T, K, E, e0, L, H, "N", N)
    got = _permute_gpu(x, ids, E, e0, L, cap)
    assert got["err"] == 0
    np.testing.assert_array_equal(got["counts"], ref["counts"])
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    np.testing.assert_array_equal(got["r2s"][:N], ref["row_to_slot"])
    np.testing.assert_array_equal(got["s2r"], ref["slot_to_row"])
    xp = to_f64(got["x_perm"])
    np.testing.assert_array_equal(xp[:N], ref["x_perm"])
    # capacity rows >= N are never written (no padding)
    assert (xp[N:] == 3.0).all() and (got["r2s"][N:] == SENT).all()
    # same result again (deterministic)
    again = _permute_gpu(x, ids, E, e0, L, cap)
    np.testing.assert_array_equal(again["r2s"], got["r2s"])
    np.testing.assert_array_equal(to_f64(again["x_perm"]), xp)


def test_permute_fp32_rows_and_duplicates():
    rng = np.random.default_rng(9)
    T, K, E, H = 300, 3, 5, 24
    ids = _rand_ids(rng, T, K, E, p_inv=0.2)
    ids[:, 1] = ids[:, 0]  # duplicate ids within a token: two rows each
    x64 = rng.standard_normal((T, H)).astype(np.float32).astype(np.float64)
    x = torch.from_numpy(x64.astype(np.float32)).to(DEV)
    ref = O.count_and_permute(ids, 0, E, x64)
    got = _permute_gpu(x, ids, E, 0, E, T * K)
    N = int(ref["offsets"][-1])
    np.testing.assert_array_equal(got["r2s"][:N], ref["row_to_slot"])
    np.testing.assert_array_equal(to_f64(got["x_perm"])[:N], ref["x_perm"])


def test_permute_mx_quantized_rows():
    rng = np.random.default_rng(10)
    T, K, E, H = 600, 2, 8, 512
    ids = _rand_ids(rng, T, K, E, distinct=True)
    x64 = O.bf16_round(rng.standard_normal((T, H)) * np.exp(rng.uniform(-8, 8, size=(T, 1))))
    ref = O.count_and_permute(ids, 0, E, x64)
    N = int(ref["offsets"][-1])
    got = _permute_gpu(bf16_from_f64(x64), ids, E, 0, E, T * K, out_dtype=D.MXFP8)
    oc, os_ = O.mx_quantize_rows(ref["x_perm"])
    np.testing.assert_array_equal(np_of(got["x_perm"])[:N], oc)
    np.testing.assert_array_equal(np_of(got["xs"])[:N], os_)
    assert (np_of(got["x_perm"])[N:] == 0x5A).all()


def test_permute_mxfp4_quantized_rows():
    rng = np.random.default_rng(11)
    T, K, E, H = 600, 2, 8, 512
    ids = _rand_ids(rng, T, K, E, distinct=True)
    x64 = O.bf16_round(rng.standard_normal((T, H)) * np.exp(rng.uniform(-8, 8, size=(T, 1))))
    x64[::11, :64] = 0.0
    ref = O.count_and_permute(ids, 0, E, x64)
    N = int(ref["offsets"][-1])
    got = _permute_gpu(bf16_from_f64(x64), ids, E, 0, E, T * K, out_dtype=D.MXFP4)
    oc, os_ = O.mx4_quantize_rows(ref["x_perm"])
    np.testing.assert_array_equal(np_of(got["x_perm"])[:N], O.pack_fp4(oc))
    np.testing.assert_array_equal(np_of(got["xs"])[:N], os_)
    assert (np_of(got["x_perm"])[N:] == 0x5A).all()


def test_permute_mxfp4_every_bf16_pattern_as_block_max():
    """Every finite bf16 value as the largest element of a block (with its
    negation, a smaller neighbour and -0 beside it), routed one row per token."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[np.isfinite(O.bits_to_bf16(bits))]
    blocks = np.zeros((bits.size, 32), np.uint16)
    blocks[:, 5] = bits
    blocks[:, 6] = bits ^ 0x8000
    blocks[:, 7] = (bits & 0x7fff) >> 1
    blocks[:, 9] = 0x8000
    x = blocks.reshape(-1, 256)  # 8 blocks per row
    T = x.shape[0]
    ids = np.zeros((T, 1), np.int16)
    say("mxfp4 exhaustive: rows", x.shape)
    xt = torch.from_numpy(x.astype(np.int16)).view(torch.bfloat16).to(DEV)
    got = _permute_gpu(xt, ids, 1, 0, 1, T, out_dtype=D.MXFP4)
    oc, os_ = O.mx4_quantize_rows(O.bits_to_bf16(x))
    np.testing.assert_array_equal(np_of(got["xs"]), os_)
    np.testing.assert_array_equal(np_of(got["x_perm"]), O.pack_fp4(oc))


def test_permute_overflow_and_bad_ids():
    rng = np.random.default_rng(11)
    T, K, E, H = 400, 2, 8, 64
    ids = _rand_ids(rng, T, K, E, p_inv=0.0)
    ref = O.count_and_permute(ids, 0, E, None)
    N = int(ref["offsets"][-1])
    cap = N - 37
    x = bf16_from_f64(O.bf16_round(rng.standard_normal((T, H))))
    got = _permute_gpu(x, ids, E, 0, E, cap)
    assert got["err"] & D.DEVERR_OVERFLOW
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])        # true counts
    np.testing.assert_array_equal(got["r2s"], ref["row_to_slot"][:cap])
    s2r = ref["slot_to_row"].copy()
    s2r[s2r >= cap] = -1
    np.testing.assert_array_equal(got["s2r"], s2r)
    bad = ids.copy()
    bad[5, 1] = 8
    bad[9, 0] = -3
    got = _permute_gpu(x, bad, E, 0, E, T * K)
    assert got["err"] & D.DEVERR_BAD_ID
    fixed = bad.copy()
    fixed[5, 1] = -1
    fixed[9, 0] = -1
    ref = O.count_and_permute(fixed, 0, E, None)
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    np.testing.assert_array_equal(got["s2r"], ref["slot_to_row"])


def test_permute_workspace_reused_across_shapes():
    """One zero-filled workspace serves calls of different shapes in a row:
    each call leaves the workspace state zero for the next."""
    rng = np.random.default_rng(13)
    E, L, H = 64, 64, 64
    ws = torch.zeros(D.moe_permute_workspace_bytes(6000, 8, L), dtype=torch.uint8, device=DEV)
    for T, K in ((6000, 8), (257, 3), (6000, 8), (1, 1), (4000, 6)):
        ids = _rand_ids(rng, T, K, E)
        x64 = O.bf16_round(rng.standard_normal((T, H)))
        ref = O.count_and_permute(ids, 0, L, x64, E_global=E)
        N = int(ref["offsets"][-1])
        say("reuse", T, K, "N", N)
        got = _permute_gpu(bf16_from_f64(x64), ids, E, 0, L, T * K, ws=ws)
        assert got["err"] == 0
        np.testing.assert_array_equal(got["offsets"], ref["offsets"])
        np.testing.assert_array_equal(got["s2r"], ref["slot_to_row"])
        np.testing.assert_array_equal(to_f64(got["x_perm"])[:N], ref["x_perm"])


def test_permute_workspace_not_zero_filled_is_reported():
    """A workspace that was not zero-filled (here: every byte 0xEE, so the
    finished-tile counter is far past the number of tiles) is reported with
    MOE_DEVERR_WORKSPACE by the host-visible error word; every workgroup ends
    normally (none waits, none scans).  After zero-filling the workspace
    again the next call is exact."""
    rng = np.random.default_rng(14)
    T, K, E, H = 3000, 8, 256, 64  # 256 local experts: the tiles' counts are scanned by the last tile
    ids = _rand_ids(rng, T, K, E)
    x64 = O.bf16_round(rng.standard_normal((T, H)))
    ws = torch.full((D.moe_permute_workspace_bytes(T, K, E),), 0xEE, dtype=torch.uint8, device=DEV)
    bad = _permute_gpu(bf16_from_f64(x64), ids, E, 0, E, T * K, ws=ws, check_ws=False)
    assert bad["err"] & D.DEVERR_WORKSPACE
    ws.zero_()
    ref = O.count_and_permute(ids, 0, E, x64, E_global=E)
    good = _permute_gpu(bf16_from_f64(x64), ids, E, 0, E, T * K, ws=ws)
    assert good["err"] == 0
    np.testing.assert_array_equal(good["offsets"], ref["offsets"])
    np.testing.assert_array_equal(good["s2r"], ref["slot_to_row"])


def test_permute_empty_and_all_invalid():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    got = _permute_gpu(x, np.zeros((0, 2), np.int16), 8, 0, 8, 0)
    assert (got["counts"] == 0).all() and (got["offsets"] == 0).all()
    x = torch.ones((50, 64), dtype=torch.bfloat16, device=DEV)
    got = _permute_gpu(x, -np.ones((50, 3), np.int16), 8, 0, 8, 150)
    assert (got["offsets"] == 0).all() and (got["s2r"] == -1).all() and (got["r2s"] == SENT).all()


# --------------------------------------------------------------------------- combine
def _combine_gpu(y, s2r, p):
    T, K = s2r.shape
    out = torch.full((T, y.shape[1]), 7.0, dtype=y.dtype, device=DEV)
    D.moe_unpermute_combine(y, torch.from_numpy(s2r.astype(np.int32)).to(DEV),
                            torch.from_numpy(p.astype(np.float32)).to(DEV), out)
    torch.cuda.synchronize()
    return to_f64(out)


# rows of 1, 2, 3-4 and more than 4 KiB pieces: 8, 4, 2 and 1 rows gathered at a time
@pytest.mark.parametrize("T,K,H,dt", [(500, 2, 4096, "bf16"), (300, 36, 512, "bf16"), (64, 8, 7168, "bf16"),
                                      (256, 2, 64, "f32"), (100, 64, 136, "bf16"), (77, 3, 1032, "f32"),
                                      (200, 6, 1024, "bf16"), (150, 5, 768, "f32"), (120, 9, 2000, "bf16")])
def test_combine_matches_oracle(T, K, H, dt):
    rng = np.random.default_rng(T * H)
    N = T * K
    s2r = rng.permutation(N).reshape(T, K)
    s2r[rng.random((T, K)) < 0.2] = -1
    s2r[0, :] = -1  # a token without any row
    p = rng.random((T, K)).astype(np.float32)
    if dt == "bf16":
        y64 = O.bf16_round(rng.standard_normal((N, H)))
        y = bf16_from_f64(y64)
    else:
        y64 = rng.standard_normal((N, H)).astype(np.float32).astype(np.float64)
        y = torch.from_numpy(y64.astype(np.float32)).to(DEV)
    got = _combine_gpu(y, s2r, p)
    want = O.combine(y64, s2r, p, dt)
    assert (got[0] == 0).all()
    assert rel_inf(got, want) <= TOL[dt]


def test_permute_then_combine_is_identity_for_k1():
    rng = np.random.default_rng(12)
    T, E, H = 1000, 6, 256
    ids = _rand_ids(rng, T, 1, E, p_inv=0.0)
    x64 = O.bf16_round(rng.standard_normal((T, H)))
    x = bf16_from_f64(x64)
    got = _permute_gpu(x, ids, E, 0, E, T)
    out = _combine_gpu(got["x_perm"], got["s2r"], np.ones((T, 1), np.float32))
    np.testing.assert_array_equal(out, x64)
