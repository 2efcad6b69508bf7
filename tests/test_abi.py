"""The C-ABI library loads without a GPU, exports every entry point declared in
include/moe.h, and rejects invalid arguments before touching HIP (these calls
pass NULL streams and pointers, so any HIP call would be visible)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    from dropless_mixture_experts_radix_amd import _lib
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(_lib.lib, n), n
    assert set(names) == set(_lib.symbols())
    assert _lib.lib.moe_abi_version() == 2


def test_status_strings():
    from dropless_mixture_experts_radix_amd import _lib
    for st in range(7):
        assert _lib.status_str(st)
    assert _lib.status_str(99) == "unknown status"


def _route(**kw):
    from dropless_mixture_experts_radix_amd import _lib
    a = dict(T=16, E=8, K=2, H=64, score=0, x_dtype=1, w_dtype=0, x=None, w=None, logits=None, bias=None,
             mask=None, ids=None, probs=None, lo=None, err=None, ws=None, wsb=0)
    a.update(kw)
    return _lib.lib.moe_route_topk(a["T"], a["E"], a["K"], a["H"], a["score"], a["x_dtype"], a["w_dtype"], a["x"],
                                   a["w"], a["logits"], a["bias"], a["mask"], a["ids"], a["probs"], a["lo"], a["err"],
                                   a["ws"], a["wsb"], None)


P = 1 << 20  # a fake, 16-byte aligned "device" address: validation never dereferences


def test_route_validation():
    assert _route(K=9) == 2          # K > E
    assert _route(K=0) == 2
    assert _route(E=5000) == 2       # E > 4096
    assert _route(K=65, E=100) == 2  # K > 64
    assert _route(score=7) == 4
    assert _route(ids=P, probs=P) == 1                     # no x / weights, no logits
    assert _route(ids=P, probs=P, x=P, w=P, H=96) == 2     # bf16 x needs H % 64 == 0
    assert _route(ids=P, probs=P, x=P, w=P, x_dtype=0, w_dtype=1) == 4
    assert _route(ids=P, probs=P, x=P + 2, w=P) == 3
    assert _route(ids=P, probs=P, x=P, w=P) == 5           # workspace missing
    assert _route(ids=P, probs=P, x=P, w=P, ws=P, wsb=16) == 5
    assert _route(T=0) == 0                                 # empty batch: a valid no-op


def _groute(**kw):
    from dropless_mixture_experts_radix_amd import _lib
    a = dict(T=16, E=256, K=8, H=64, ng=8, tg=4, scale=1.0, x_dtype=1, w_dtype=1, x=None, w=None, logits=P,
             bias=None, mask=None, ids=P, probs=P, lo=None, so=None, err=None, ws=None, wsb=0)
    a.update(kw)
    return _lib.lib.moe_route_topk_grouped(a["T"], a["E"], a["K"], a["H"], a["ng"], a["tg"], a["scale"],
                                           a["x_dtype"], a["w_dtype"], a["x"], a["w"], a["logits"], a["bias"],
                                           a["mask"], a["ids"], a["probs"], a["lo"], a["so"], a["err"], a["ws"],
                                           a["wsb"], None)


def test_grouped_route_validation():
    assert _groute(T=0) == 0                  # empty batch: a valid no-op
    assert _groute(E=32, ng=4, tg=2, K=4) == 2   # E <= 32: no grouped path
    assert _groute(E=2048) == 2               # E > 1024
    assert _groute(ng=7) == 2                 # n_group does not divide E
    assert _groute(ng=128, E=512) == 2        # n_group > 64
    assert _groute(tg=0) == 2
    assert _groute(tg=9) == 2                 # topk_group > n_group
    assert _groute(tg=3) == 2                 # topk_group does not divide K
    assert _groute(K=36, tg=4) == 2           # K / topk_group > 8
    assert _groute(E=64, ng=32, tg=4, K=12) == 2  # K / topk_group > E / n_group
    assert _groute(scale=0.0) == 2
    assert _groute(scale=float("nan")) == 2
    assert _groute(so=P + 4) == 3             # scores_out not 16-byte aligned
    assert _groute(ids=None) == 1
    assert _groute(logits=None, x=P, w=P) == 5   # projection needs the workspace


def test_backward_validation():
    from dropless_mixture_experts_radix_amd import _lib
    L = _lib.lib
    # combine backward: (T, K, H, dtype, dout, y, s2r, probs, d_y, d_probs, stream)
    cb = L.moe_unpermute_combine_backward
    assert cb(0, 2, 64, 1, None, None, None, None, None, None, None, None, None) == 0
    assert cb(4, 2, 60, 1, P, P, P, P, P, P, None, None, None) == 2   # H % 8
    assert cb(4, 2, 64, 3, P, P, P, P, P, P, None, None, None) == 4   # dtype
    assert cb(4, 2, 64, 1, P, P, P, None, P, P, None, None, None) == 1
    assert cb(4, 2, 64, 1, P + 8, P, P, P, P, P, None, None, None) == 3
    # the MX form of d_y: bf16 rows only, H % 32, both pointers, codes 16-byte aligned
    assert cb(4, 2, 64, 0, P, P, P, P, P, P, P, P, None) == 4
    assert cb(4, 2, 48, 1, P, P, P, P, P, P, P, P, None) == 2
    assert cb(4, 2, 64, 1, P, P, P, P, P, P, P, None, None) == 1
    assert cb(4, 2, 64, 1, P, P, P, P, P, P, P + 4, P, None) == 3
    # permute backward: (T, K, H, dtype, d_x_perm, s2r, d_x, stream)
    assert L.moe_permute_backward(0, 2, 64, 1, None, None, None, None) == 0
    assert L.moe_permute_backward(4, 65, 64, 1, P, P, P, None) == 2
    assert L.moe_permute_backward(4, 2, 64, 1, P, None, P, None) == 1
    assert L.moe_permute_backward(4, 2, 64, 1, P, P, P + 4, None) == 3
    # route backward: (T, E, K, score, scale, ids, probs, d_probs, logits, bias, d_z, stream)
    assert L.moe_route_backward(0, 8, 2, 0, 1.0, None, None, None, None, None, None, None) == 0
    assert L.moe_route_backward(4, 8, 9, 0, 1.0, P, P, P, None, None, P, None) == 2    # K > E
    assert L.moe_route_backward(4, 8, 2, 5, 1.0, P, P, P, None, None, P, None) == 4    # score
    assert L.moe_route_backward(4, 8, 2, 0, 0.0, P, P, P, None, None, P, None) == 2    # scale
    assert L.moe_route_backward(4, 8, 2, 0, 1.0, P, None, P, None, None, P, None) == 1  # softmax needs probs
    assert L.moe_route_backward(4, 8, 2, 1, 1.0, P, P, P, None, None, P, None) == 1    # sigmoid needs logits
    # backward panels: (L, H, F, dtype, w1, w2, w1t, w2t, w1t_s, w2t_s, stream)
    assert L.moe_prepare_weights_backward(2, 256, 128, 2, P, P, P, P, P, P, None) == 2   # MXFP8: F % 256
    assert L.moe_prepare_weights_backward(2, 256, 256, 2, P, P, P, P, None, P, None) == 1  # MXFP8 needs scales
    assert L.moe_prepare_weights_backward(2, 256, 256, 3, P, P, P, P, P, P, None) == 4   # MXFP4: no panels
    # data gradient: (L, H, F, cap, dtype, x, offs, w1p, w1p_s, w1t, w1t_s, w2t, w2t_s, d_y, d_x, ws, wsb, stream)
    dg = lambda dt, H=256, F=256, s=P, wsb=1 << 30, xq=None, xqs=None, dq=None, dqs=None, x=P, dy=P: \
        L.moe_grouped_mlp_backward_data(2, H, F, 64, dt, x, P, P, s, P, s, P, s, dy, P, xq, xqs, dq, dqs, P, wsb, None)
    assert dg(3) == 4                       # MXFP4
    assert dg(2, F=128) == 2                # MXFP8: F % 256
    assert dg(2, s=None) == 1               # MXFP8 needs the scales
    assert dg(2, wsb=L.moe_grouped_mlp_backward_workspace_bytes(64, 256, 256, 2) - 1) == 5
    # row-wise MX operands from their producers: MXFP8 only, codes and scales together, then the bf16 operand
    # may be absent; scales 4-byte aligned
    assert dg(1, H=256, F=256, s=None, xq=P, xqs=P) == 4
    assert dg(2, xq=P) == 1
    assert dg(2, dqs=P) == 1
    assert dg(2, x=None) == 1
    assert dg(2, xq=P, xqs=P + 2) == 3
    assert dg(2, dq=P + 8, dqs=P) == 3
    assert (L.moe_grouped_mlp_backward_workspace_bytes(64, 256, 256, 2) >
            L.moe_grouped_mlp_backward_workspace_bytes(64, 256, 256, 1))
    assert L.moe_prepared_weight_bytes(2, 256, 512, 2, 7) == 2 * 256 * 2 * 16   # W1t scales
    assert L.moe_prepared_weight_bytes(2, 256, 512, 2, 8) == 2 * 512 * 1 * 16   # W2t scales


def test_permute_validation():
    from dropless_mixture_experts_radix_amd import _lib
    f = _lib.lib.moe_permute

    def call(T=4, H=64, K=2, E=8, e0=0, L=8, cap=8, xd=1, od=1, x=P, ids=P, counts=P, offs=P, xp=P, xs=None,
             r2s=P, s2r=P, ws=P, wsb=1 << 20):
        return f(T, H, K, E, e0, L, cap, xd, od, x, ids, counts, offs, xp, xs, r2s, s2r, None, ws, wsb, None)

    assert call(e0=4, L=8) == 2          # local range beyond E
    assert call(K=65) == 2
    assert call(E=40000, L=8) == 2
    assert call(L=3000, E=4000) == 2     # L > MOE_MAX_L
    assert call(xd=0, od=2) == 4         # MX output needs bf16 rows
    assert call(od=2, H=48) == 2         # MX needs H % 32 == 0
    assert call(od=2) == 1               # MX scales missing
    assert call(xd=0, od=3) == 4         # MXFP4 output needs bf16 rows
    assert call(od=3, H=48) == 2
    assert call(od=3) == 1
    assert call(counts=None) == 1
    assert call(ws=None) == 5
    assert call(wsb=8) == 5
    assert call(x=P + 8) == 3
    assert call(H=12) == 2               # bf16 rows need H % 8 == 0


def test_mlp_validation():
    from dropless_mixture_experts_radix_amd import _lib
    f = _lib.lib.moe_grouped_mlp

    def call(L=8, H=128, F=128, cap=64, dt=1, x=P, xs=None, offs=P, w1=P, w1s=None, w2=P, w2s=None, y=P, ws=P,
             wsb=1 << 24):
        return f(L, H, F, cap, dt, x, xs, offs, w1, w1s, w2, w2s, y, ws, wsb, None)

    assert call(H=96) == 2               # bf16 needs H % 128 == 0
    assert call(H=192) == 2
    assert call(dt=2, F=384) == 2        # MXFP8 needs F % 256 == 0
    assert call(dt=2, H=256, F=256) == 1  # MX scales missing
    assert call(dt=3, H=512, F=768) == 2  # MXFP4 needs F % 512 == 0
    assert call(dt=3, H=256, F=512) == 2  # ... and H % 512 == 0
    assert call(dt=3, H=512, F=512) == 1
    assert call(dt=3, H=512, F=512, xs=P, w1s=P + 2, w2s=P) == 3  # scale pointers 4-byte aligned
    assert call(dt=9) == 4
    assert call(offs=None) == 1
    assert call(wsb=100) == 5
    assert call(L=0) == 2
    assert call(y=P + 4) == 3


def test_other_validation():
    from dropless_mixture_experts_radix_amd import _lib
    lib = _lib.lib
    assert lib.moe_unpermute_combine(4, 2, 12, 1, P, P, P, P, None) == 2      # H % 8
    assert lib.moe_unpermute_combine(4, 2, 64, 2, P, P, P, P, None) == 4      # MX output not supported
    assert lib.moe_unpermute_combine(4, 2, 64, 1, P, None, P, P, None) == 1
    assert lib.moe_mx_quantize(4, 48, P, None, P, P, None) == 2
    assert lib.moe_mx_quantize(4, 64, None, None, P, P, None) == 1
    assert lib.moe_prepare_weights(2, 64, 48, 1, 1, P, P, P, P, None, None, None) == 2   # F % 32
    assert lib.moe_prepare_weights(2, 256, 256, 0, 2, P, P, P, P, P, P, None) == 4       # MX from fp32
    assert lib.moe_prepare_weights(2, 256, 384, 1, 2, P, P, P, P, P, P, None) == 2       # MX needs F % 256
    assert lib.moe_prepare_weights(2, 256, 256, 1, 2, P, P, P, P, None, P, None) == 1
    assert lib.moe_prepare_weights(2, 512, 768, 1, 3, P, P, P, P, P, P, None) == 2       # MXFP4 needs F % 512
    assert lib.moe_prepare_weights(2, 512, 512, 0, 3, P, P, P, P, P, P, None) == 4
    assert lib.moe_prepare_router(P, 1, 0, 64, 8, P, None) == 4                          # bf16 W_r, fp32 x
    assert lib.moe_prepare_router(None, 0, 1, 64, 8, P, None) == 1


def test_size_queries():
    from dropless_mixture_experts_radix_amd import _lib
    lib = _lib.lib
    # fp32 router weights for bf16 rows: 3 bf16 terms per weight, 10 experts per 32-row tile
    assert lib.moe_router_prepared_bytes(4096, 8, 0, 1) == 32 * 4096 * 2
    assert lib.moe_router_prepared_bytes(7168, 256, 1, 1) == 256 * 7168 * 2
    assert lib.moe_router_prepared_bytes(64, 8, 0, 0) == 64 * 8 * 4
    assert lib.moe_prepared_weight_bytes(8, 4096, 14336, 1, 1) == 8 * 2 * 14336 * 4096 * 2
    assert lib.moe_prepared_weight_bytes(8, 4096, 14336, 2, 3) == 8 * 2 * 14336 * 4096 // 32
    # MX scales: 16 bytes per prepared row and 512-wide k group (short last group padded)
    assert lib.moe_prepared_weight_bytes(2, 768, 256, 2, 3) == 2 * 512 * 2 * 16
    assert lib.moe_prepared_weight_bytes(2, 768, 256, 2, 4) == 2 * 768 * 1 * 16
    assert lib.moe_prepared_weight_bytes(8, 4096, 14336, 1, 3) == 0
    # MXFP4: codes two per byte, scales as for MXFP8
    assert lib.moe_prepared_weight_bytes(8, 4096, 14336, 3, 1) == 8 * 2 * 14336 * 4096 // 2
    assert lib.moe_prepared_weight_bytes(2, 1024, 512, 3, 2) == 2 * 1024 * 512 // 2
    assert lib.moe_prepared_weight_bytes(2, 1024, 512, 3, 3) == lib.moe_prepared_weight_bytes(2, 1024, 512, 2, 3)
    assert (lib.moe_grouped_mlp_workspace_bytes(8192, 14336, 3) <
            lib.moe_grouped_mlp_workspace_bytes(8192, 14336, 2))
    assert lib.moe_grouped_mlp_workspace_bytes(8192, 14336, 1) >= 8192 * 14336 * 2
    assert lib.moe_permute_workspace_bytes(8192, 36, 32) >= 8192 * 36 * 4


def test_query_sizes():
    """moe_query_sizes agrees with the per-buffer size functions, gives the exact
    routed-row bounds T*min(K, L) and T*K, and rejects bad shapes (host only)."""
    from dropless_mixture_experts_radix_amd import _lib
    lib = _lib.lib
    q = lambda **kw: _lib.moe_query_sizes(**kw)
    z = q(T=4096, H=4096, E=8, K=2, F=14336, dtype=1, x_dtype=1, w_dtype=0)
    assert z["capacity"] == 8192 and z["capacity_any_ids"] == 8192
    assert z["router_prepared_bytes"] == lib.moe_router_prepared_bytes(4096, 8, 0, 1)
    assert z["route_workspace_bytes"] == lib.moe_route_workspace_bytes(4096, 8, 4096, 1)
    assert z["permute_workspace_bytes"] == lib.moe_permute_workspace_bytes(4096, 2, 8)
    assert z["mlp_workspace_bytes"] == lib.moe_grouped_mlp_workspace_bytes(8192, 14336, 1)
    assert z["w1p_bytes"] == lib.moe_prepared_weight_bytes(8, 4096, 14336, 1, 1)
    assert z["w1t_bytes"] == lib.moe_prepared_weight_bytes(8, 4096, 14336, 1, 5)
    assert z["mlp_backward_workspace_bytes"] == lib.moe_grouped_mlp_backward_workspace_bytes(8192, 4096, 14336, 1)
    assert z["bwd_dh_offset"] == (8192 * 2 * 14336 * 2 + 255) // 256 * 256 and z["bwd_dh_codes_offset"] == 0
    # sparse share: 32 local experts of 2304, K = 36 > L
    z = q(T=8192, H=512, E=2304, K=36, L=32, F=512, dtype=1)
    assert z["capacity"] == 8192 * 32 and z["capacity_any_ids"] == 8192 * 36
    # MXFP8: the MX activations' scales follow the codes; d_h's MX operands sit inside the backward workspace
    z = q(T=4096, H=4096, E=8, K=2, F=14336, dtype=2)
    assert z["mlp_act_scales_offset"] == 8192 * 14336
    assert 0 < z["bwd_dh_codes_offset"] < z["bwd_dh_scales_offset"]
    assert z["bwd_dh_scales_offset"] + 8192 * 2 * 14336 // 32 <= z["mlp_backward_workspace_bytes"]
    assert z["w1p_scales_bytes"] == lib.moe_prepared_weight_bytes(8, 4096, 14336, 2, 3)
    # MXFP4 has no backward panels
    z = q(T=64, H=512, E=8, K=2, F=512, dtype=3)
    assert z["w1t_bytes"] == 0 and z["mlp_backward_workspace_bytes"] == 0
    for bad in (dict(K=9), dict(K=0), dict(E=5000), dict(L=9), dict(T=-1)):
        kw = dict(T=16, H=64, E=8, K=2, F=128, dtype=1)
        kw.update(bad)
        with pytest.raises(_lib.MoEError):
            q(**kw)
    with pytest.raises(_lib.MoEError):
        q(T=16, H=64, E=8, K=2, F=128, dtype=7)
    assert lib.moe_query_sizes(None, None) == 1


def test_mlp_with_act_validation():
    from dropless_mixture_experts_radix_amd import _lib
    f = _lib.lib.moe_grouped_mlp_with_act

    def call(dt=2, H=256, F=256, xs=P, w1s=P, w2s=P, act=P, wsb=1 << 28):
        return f(8, H, F, 64, dt, P, xs, P, P, w1s, P, w2s, P, P, wsb, act, None)

    assert call(act=None) == 1           # the hook's output is required
    assert call(dt=1, H=128, F=128) == 4  # bf16: `a` is in the workspace already
    assert call(act=P + 8) == 3
    assert call(w2s=P + 1) == 3


def test_backward_scale_alignment():
    """The MXFP8 data gradient reads its weight scales 4 bytes at a time, as the
    forward does: misaligned scale pointers are rejected."""
    from dropless_mixture_experts_radix_amd import _lib
    L = _lib.lib
    dg = lambda s1=P, s2=P, s3=P: L.moe_grouped_mlp_backward_data(2, 256, 256, 64, 2, P, P, P, s1, P, s2, P, s3, P,
                                                                   P, None, None, None, None, P, 1 << 30, None)
    assert dg(s1=P + 2) == 3
    assert dg(s2=P + 1) == 3
    assert dg(s3=P + 3) == 3
