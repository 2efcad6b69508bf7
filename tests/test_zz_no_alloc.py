"""moe_permute_noalloc (the permute for callers that cannot allocate: its
workspace is a fixed device array of the library) against moe_permute with a
caller workspace, through the C ABI: bit-exact counts, offsets, maps, rows and
error word on two calls in a row, the second with a smaller input, plus the
limit check."""
import ctypes

import numpy as np
import pytest
import torch

import dropless_mixture_experts_radix_amd as D
from dropless_mixture_experts_radix_amd import _lib
from oracle import moe_oracle as O
from tests.gpu_util import DEV, bf16_from_f64, np_of, say, to_f64

pytestmark = pytest.mark.gpu

SENT = -555


def _outputs(T, H, K, L, cap):
    return dict(counts=torch.full((L,), SENT, dtype=torch.int32, device=DEV),
                offsets=torch.full((L + 1,), SENT, dtype=torch.int32, device=DEV),
                x_perm=torch.full((cap, H), 3.0, dtype=torch.bfloat16, device=DEV),
                r2s=torch.full((cap,), SENT, dtype=torch.int32, device=DEV),
                s2r=torch.full((T, K), SENT, dtype=torch.int32, device=DEV),
                err=torch.zeros(1, dtype=torch.int32, device=DEV))


def _call(fn, x, ids, E, e0, L, o, extra):
    T, H = x.shape
    K = ids.shape[1]
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = fn(T, H, K, E, e0, L, o["r2s"].shape[0], D.BF16, D.BF16, p(x), p(ids), p(o["counts"]), p(o["offsets"]),
            p(o["x_perm"]), None, p(o["r2s"]), p(o["s2r"]), p(o["err"]), *extra,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, _lib.status_str(st)


def test_permute_noalloc_matches_permute_two_calls():
    lib = _lib.lib
    rng = np.random.default_rng(21)
    E, e0, L, H = 2304, 0, 32, 256
    for T, K in ((8192, 36), (1000, 9)):   # the second call smaller than the first
        ids64 = np.where(rng.random((T, K)) < 0.1, -1, rng.integers(0, 40, size=(T, K)))
        ids = torch.from_numpy(ids64.astype(np.int16)).to(DEV)
        x64 = O.bf16_round(rng.standard_normal((T, H)))
        x = bf16_from_f64(x64)
        cap = T * K
        a, b = _outputs(T, H, K, L, cap), _outputs(T, H, K, L, cap)
        ws = torch.zeros(D.moe_permute_workspace_bytes(T, K, L), dtype=torch.uint8, device=DEV)
        say("noalloc permute T", T, "K", K)
        _call(lib.moe_permute, x, ids, E, e0, L, a, [ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel())])
        _call(lib.moe_permute_noalloc, x, ids, E, e0, L, b, [])
        torch.cuda.synchronize()
        for k in ("counts", "offsets", "r2s", "s2r", "err"):
            np.testing.assert_array_equal(np_of(b[k]), np_of(a[k]), err_msg=k)
        np.testing.assert_array_equal(to_f64(b["x_perm"]), to_f64(a["x_perm"]))
        ref = O.count_and_permute(ids64.astype(np.int16), e0, L, x64, E_global=E)
        np.testing.assert_array_equal(np_of(b["offsets"]), ref["offsets"])
        assert int(b["err"].item()) == 0
    # a shape whose workspace exceeds the fixed array is refused before any launch
    big_T = 1 << 20
    assert D.moe_permute_workspace_bytes(big_T, 64, 2048) > lib.moe_permute_noalloc_max_workspace_bytes()
    P = 1 << 20
    st = lib.moe_permute_noalloc(big_T, 64, 8, 4096, 0, 2048, big_T * 8, D.BF16, D.BF16, P, P, P, P, P, None, P, P,
                                 None, None)
    assert st == 5  # MOE_ERR_WORKSPACE
