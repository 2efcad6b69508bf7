"""ctypes binding of libmoe_mi355x.so (the C ABI in include/moe.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their data pointers, shapes and the current HIP stream
to the library, and raises MoEError on a non-zero status.  No computation of
the layer happens here.  Loading fails loudly when the library is missing.
"""
import ctypes
import os

import torch

F32, BF16, MXFP8, MXFP4 = 0, 1, 2, 3
SOFTMAX, SIGMOID = 0, 1
DEVERR_BAD_ID, DEVERR_OVERFLOW, DEVERR_NONFINITE, DEVERR_WORKSPACE = 1, 2, 4, 8
MAX_K, MAX_E, MAX_L = 64, 4096, 2048

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

_I, _I64, _SZ, _P = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

class MoeShape(ctypes.Structure):
    """moe_shape of include/moe.h."""
    _fields_ = [(n, _I) for n in ("T", "H", "E", "K", "L", "F", "x_dtype", "w_dtype", "dtype")]


class MoeSizes(ctypes.Structure):
    """moe_sizes of include/moe.h."""
    _fields_ = ([("capacity", _I64), ("capacity_any_ids", _I64)] +
                [(n, _SZ) for n in ("router_prepared_bytes", "route_workspace_bytes", "permute_workspace_bytes",
                                    "permute_state_bytes", "w1p_bytes", "w2p_bytes", "w1p_scales_bytes", "w2p_scales_bytes",
                                    "mlp_workspace_bytes", "mlp_act_offset", "mlp_act_scales_offset",
                                    "w1t_bytes", "w2t_bytes", "w1t_scales_bytes", "w2t_scales_bytes",
                                    "mlp_backward_workspace_bytes", "bwd_h_offset", "bwd_dh_offset",
                                    "bwd_dh_codes_offset", "bwd_dh_scales_offset",
                                    "mlp_backward_weights_workspace_bytes")])


_SIGS = {
    "moe_abi_version": (_I, []),
    "moe_query_sizes": (_I, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeSizes)]),
    "moe_grouped_mlp_with_act": (_I, [_I, _I, _I, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "moe_calib_copy": (_I, [_P, _P, _SZ, _P]),
    "moe_calib_read_out_words": (_SZ, [_SZ]),
    "moe_calib_read": (_I, [_P, _SZ, _P, _P]),
    "moe_calib_write": (_I, [_P, _SZ, ctypes.c_uint32, _P]),
    "moe_calib_mfma": (_I, [_I, _I, _I, _P, _P]),
    "moe_status_str": (ctypes.c_char_p, [_I]),
    "moe_router_prepared_bytes": (_SZ, [_I, _I, _I, _I]),
    "moe_prepare_router": (_I, [_P, _I, _I, _I, _I, _P, _P]),
    "moe_route_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "moe_route_topk": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_topk_grouped": (_I, [_I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _P, _P, _P, _SZ, _P]),
    "moe_permute_workspace_bytes": (_SZ, [_I, _I, _I]),
    "moe_permute": (_I, [_I, _I, _I, _I, _I, _I, _I64, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute_noalloc_max_workspace_bytes": (_SZ, []),
    "moe_permute_noalloc": (_I, [_I, _I, _I, _I, _I, _I, _I64, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_prepared_weight_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "moe_prepare_weights": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_mlp_workspace_bytes": (_SZ, [_I64, _I, _I]),
    "moe_grouped_mlp": (_I, [_I, _I, _I, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_unpermute_combine": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "moe_mx_quantize": (_I, [_I64, _I, _P, _P, _P, _P, _P]),
    "moe_unpermute_combine_backward": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_prepare_weights_backward": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_mlp_backward_workspace_bytes": (_SZ, [_I64, _I, _I, _I]),
    "moe_grouped_mlp_backward_data": (_I, [_I, _I, _I, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, _SZ, _P]),
    "moe_grouped_mlp_backward_weights_workspace_bytes": (_SZ, [_I, _I64, _I, _I, _I]),
    "moe_mx_columns_grouped_max_blocks": (_I64, [_I, _I64]),
    "moe_mx_quantize_columns_grouped": (_I, [_I, _I64, _I, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_mlp_backward_weights": (_I, [_I, _I, _I, _I64, _I, _P, _P, _P, _P, _SZ, _P, _P, _P, _SZ, _P]),
    "moe_permute_backward": (_I, [_I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_route_backward": (_I, [_I, _I, _I, _I, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P]),
}


class MoEError(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m dropless_mixture_experts_radix_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe_abi_version() != 2:
        raise ImportError("libmoe_mi355x.so ABI version mismatch")
    return lib


lib = _load()


def symbols():
    return list(_SIGS)


def status_str(st: int) -> str:
    return lib.moe_status_str(st).decode()


def _check(st, name):
    if st != 0:
        raise MoEError(f"{name}: {status_str(st)} (status {st})")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def dtype_code(t: torch.dtype) -> int:
    return {torch.float32: F32, torch.bfloat16: BF16, torch.uint8: MXFP8}[t]


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


# ----------------------------------------------------------------- route
def moe_router_prepared_bytes(H, E, w_dtype, x_dtype):
    return lib.moe_router_prepared_bytes(H, E, w_dtype, x_dtype)


def moe_prepare_router(w_router, x_dtype, prepared):
    H, E = w_router.shape
    _check(lib.moe_prepare_router(_p(w_router), dtype_code(w_router.dtype), x_dtype, H, E, _p(prepared),
                                  _stream()), "moe_prepare_router")


def moe_route_workspace_bytes(T, E, H, x_dtype):
    return lib.moe_route_workspace_bytes(T, E, H, x_dtype)


def moe_route_topk(ids, probs, score, *, logits=None, x=None, w_prepared=None, w_dtype=F32, E=None,
                   bias=None, mask=None, logits_out=None, err=None, workspace=None):
    T, K = ids.shape
    if logits is not None:
        E = logits.shape[1]
        H, x_dtype = 0, F32
    else:
        H = x.shape[1]
        x_dtype = dtype_code(x.dtype)
    _check(lib.moe_route_topk(T, E, K, H, score, x_dtype, w_dtype, _p(x), _p(w_prepared), _p(logits), _p(bias),
                              _p(mask), _p(ids), _p(probs), _p(logits_out), _p(err), _p(workspace),
                              _nbytes(workspace), _stream()), "moe_route_topk")


def moe_route_topk_grouped(ids, probs, n_group, topk_group, scale=1.0, *, logits=None, x=None, w_prepared=None,
                           w_dtype=F32, E=None, bias=None, mask=None, logits_out=None, scores_out=None, err=None,
                           workspace=None):
    T, K = ids.shape
    if logits is not None:
        E = logits.shape[1]
        H, x_dtype = 0, F32
    else:
        H = x.shape[1]
        x_dtype = dtype_code(x.dtype)
    _check(lib.moe_route_topk_grouped(T, E, K, H, n_group, topk_group, float(scale), x_dtype, w_dtype, _p(x),
                                      _p(w_prepared), _p(logits), _p(bias), _p(mask), _p(ids), _p(probs),
                                      _p(logits_out), _p(scores_out), _p(err), _p(workspace), _nbytes(workspace),
                                      _stream()), "moe_route_topk_grouped")


# ----------------------------------------------------------------- permute
def moe_permute_workspace_bytes(T, K, L):
    return lib.moe_permute_workspace_bytes(T, K, L)


def moe_permute(x, ids, E_global, e0, L, counts, offsets, x_perm, row_to_slot, slot_to_row, workspace,
                x_perm_scales=None, err=None, out_dtype=None):
    T, H = x.shape
    K = ids.shape[1]
    capacity = row_to_slot.shape[0]
    x_dtype = dtype_code(x.dtype)
    out_dtype = x_dtype if out_dtype is None else out_dtype
    _check(lib.moe_permute(T, H, K, E_global, e0, L, capacity, x_dtype, out_dtype, _p(x), _p(ids), _p(counts),
                           _p(offsets), _p(x_perm), _p(x_perm_scales), _p(row_to_slot), _p(slot_to_row), _p(err),
                           _p(workspace), _nbytes(workspace), _stream()), "moe_permute")


def moe_permute_noalloc(x, ids, E_global, e0, L, counts, offsets, x_perm, row_to_slot, slot_to_row,
                        x_perm_scales=None, err=None, out_dtype=None):
    """moe_permute with the library's fixed device workspace (allocates nothing)."""
    T, H = x.shape
    K = ids.shape[1]
    capacity = row_to_slot.shape[0]
    x_dtype = dtype_code(x.dtype)
    out_dtype = x_dtype if out_dtype is None else out_dtype
    _check(lib.moe_permute_noalloc(T, H, K, E_global, e0, L, capacity, x_dtype, out_dtype, _p(x), _p(ids),
                                   _p(counts), _p(offsets), _p(x_perm), _p(x_perm_scales), _p(row_to_slot),
                                   _p(slot_to_row), _p(err), _stream()), "moe_permute_noalloc")


# ----------------------------------------------------------------- weights
def moe_prepared_weight_bytes(L, H, F, dtype, which):
    return lib.moe_prepared_weight_bytes(L, H, F, dtype, which)


def moe_prepare_weights(w1, w2, dtype, w1p, w2p, w1p_scales=None, w2p_scales=None):
    L, H, F2 = w1.shape
    _check(lib.moe_prepare_weights(L, H, F2 // 2, dtype_code(w1.dtype), dtype, _p(w1), _p(w2), _p(w1p), _p(w2p),
                                   _p(w1p_scales), _p(w2p_scales), _stream()), "moe_prepare_weights")


# ----------------------------------------------------------------- grouped MLP
def moe_grouped_mlp_workspace_bytes(capacity, F, dtype):
    return lib.moe_grouped_mlp_workspace_bytes(capacity, F, dtype)


def moe_grouped_mlp(x_perm, offsets, w1p, w2p, y_perm, workspace, dtype, H, F, x_perm_scales=None,
                    w1p_scales=None, w2p_scales=None):
    L = offsets.shape[0] - 1
    capacity = y_perm.shape[0]
    _check(lib.moe_grouped_mlp(L, H, F, capacity, dtype, _p(x_perm), _p(x_perm_scales), _p(offsets), _p(w1p),
                               _p(w1p_scales), _p(w2p), _p(w2p_scales), _p(y_perm), _p(workspace),
                               _nbytes(workspace), _stream()), "moe_grouped_mlp")


def moe_grouped_mlp_with_act(x_perm, offsets, w1p, w2p, y_perm, workspace, dtype, H, F, act_bf16,
                             x_perm_scales=None, w1p_scales=None, w2p_scales=None):
    """moe_grouped_mlp (MX dtypes) that also stores the bf16 `a` its GEMM1
    epilogue quantizes into act_bf16 [capacity][F] (a test hook)."""
    L = offsets.shape[0] - 1
    capacity = y_perm.shape[0]
    _check(lib.moe_grouped_mlp_with_act(L, H, F, capacity, dtype, _p(x_perm), _p(x_perm_scales), _p(offsets),
                                        _p(w1p), _p(w1p_scales), _p(w2p), _p(w2p_scales), _p(y_perm),
                                        _p(workspace), _nbytes(workspace), _p(act_bf16), _stream()),
           "moe_grouped_mlp_with_act")


# ----------------------------------------------------------------- calibration kernels
def moe_calib_copy(src, dst):
    n = min(_nbytes(src), _nbytes(dst)) // 16 * 16
    _check(lib.moe_calib_copy(_p(src), _p(dst), n, _stream()), "moe_calib_copy")
    return n


def moe_calib_read(src, out):
    n = _nbytes(src) // 16 * 16
    if out.numel() < lib.moe_calib_read_out_words(n):
        raise MoEError("moe_calib_read: out too small")
    _check(lib.moe_calib_read(_p(src), n, _p(out), _stream()), "moe_calib_read")
    return n


def moe_calib_read_out_words(nbytes):
    return lib.moe_calib_read_out_words(nbytes)


def moe_calib_write(dst, value=0):
    n = _nbytes(dst) // 16 * 16
    _check(lib.moe_calib_write(_p(dst), n, value, _stream()), "moe_calib_write")
    return n


def moe_calib_mfma(dtype, blocks, iters, out):
    if out.numel() < blocks * 512:
        raise MoEError("moe_calib_mfma: out too small")
    _check(lib.moe_calib_mfma(dtype, blocks, iters, _p(out), _stream()), "moe_calib_mfma")
    return blocks * 8 * 4 * iters * (32768 if dtype == BF16 else 131072)


# ----------------------------------------------------------------- sizes
def moe_query_sizes(T, H, E, K, F, dtype, x_dtype=BF16, w_dtype=F32, L=0):
    """All buffer sizes of one layer shape (moe_query_sizes), as a dict."""
    sh = MoeShape(T, H, E, K, L, F, x_dtype, w_dtype, dtype)
    out = MoeSizes()
    _check(lib.moe_query_sizes(ctypes.byref(sh), ctypes.byref(out)), "moe_query_sizes")
    return {n: getattr(out, n) for n, _ in MoeSizes._fields_}


# ----------------------------------------------------------------- combine
def moe_unpermute_combine(y_perm, slot_to_row, probs, out):
    T, K = slot_to_row.shape
    H = out.shape[1]
    _check(lib.moe_unpermute_combine(T, K, H, dtype_code(out.dtype), _p(y_perm), _p(slot_to_row), _p(probs),
                                     _p(out), _stream()), "moe_unpermute_combine")


# ----------------------------------------------------------------- MX quantizer
def moe_mx_quantize(inp, codes, scales, row_limit=None):
    rows, cols = inp.shape
    _check(lib.moe_mx_quantize(rows, cols, _p(inp), _p(row_limit), _p(codes), _p(scales), _stream()),
           "moe_mx_quantize")


# ----------------------------------------------------------------- backward
def _need(t, dtype, name):
    if t is not None and t.dtype != dtype:
        raise MoEError(f"{name} must be {dtype}, got {t.dtype}")


def moe_unpermute_combine_backward(dout, y_perm, slot_to_row, probs, d_y_perm, d_probs, d_y_perm_q=None,
                                   d_y_perm_q_scales=None):
    _need(slot_to_row, torch.int32, "slot_to_row")
    _need(probs, torch.float32, "probs")
    _need(d_probs, torch.float32, "d_probs")
    T, K = slot_to_row.shape
    H = dout.shape[1]
    _check(lib.moe_unpermute_combine_backward(T, K, H, dtype_code(dout.dtype), _p(dout), _p(y_perm),
                                              _p(slot_to_row), _p(probs), _p(d_y_perm), _p(d_probs),
                                              _p(d_y_perm_q), _p(d_y_perm_q_scales), _stream()),
           "moe_unpermute_combine_backward")


def moe_permute_backward(d_x_perm, slot_to_row, d_x):
    _need(slot_to_row, torch.int32, "slot_to_row")
    T, K = slot_to_row.shape
    H = d_x.shape[1]
    _check(lib.moe_permute_backward(T, K, H, dtype_code(d_x.dtype), _p(d_x_perm), _p(slot_to_row), _p(d_x),
                                    _stream()), "moe_permute_backward")


def moe_route_backward(ids, d_probs, d_z, score, *, probs=None, logits=None, score_bias=None, scale=1.0, E=None):
    _need(ids, torch.int16, "ids")
    for t, n in ((d_probs, "d_probs"), (d_z, "d_z"), (probs, "probs"), (logits, "logits"), (score_bias, "score_bias")):
        _need(t, torch.float32, n)
    T, K = ids.shape
    if logits is not None:
        E = logits.shape[1]
    _check(lib.moe_route_backward(T, E, K, score, float(scale), _p(ids), _p(probs), _p(d_probs), _p(logits),
                                  _p(score_bias), _p(d_z), _stream()), "moe_route_backward")


def moe_prepare_weights_backward(w1, w2, w1t, w2t, w1t_scales=None, w2t_scales=None, dtype=BF16):
    L, H, F2 = w1.shape
    _check(lib.moe_prepare_weights_backward(L, H, F2 // 2, dtype, _p(w1), _p(w2), _p(w1t), _p(w2t), _p(w1t_scales),
                                            _p(w2t_scales), _stream()), "moe_prepare_weights_backward")


def moe_grouped_mlp_backward_workspace_bytes(capacity, H, F, dtype):
    return lib.moe_grouped_mlp_backward_workspace_bytes(capacity, H, F, dtype)


def moe_grouped_mlp_backward_data(x_perm, offsets, w1p, w1t, w2t, d_y_perm, d_x_perm, workspace, H, F, dtype=BF16,
                                  w1p_scales=None, w1t_scales=None, w2t_scales=None, x_perm_q=None,
                                  x_perm_q_scales=None, d_y_perm_q=None, d_y_perm_q_scales=None):
    _need(offsets, torch.int32, "offsets")
    L = offsets.shape[0] - 1
    cap = d_x_perm.shape[0]
    _check(lib.moe_grouped_mlp_backward_data(L, H, F, cap, dtype, _p(x_perm), _p(offsets), _p(w1p), _p(w1p_scales),
                                             _p(w1t), _p(w1t_scales), _p(w2t), _p(w2t_scales), _p(d_y_perm),
                                             _p(d_x_perm), _p(x_perm_q), _p(x_perm_q_scales), _p(d_y_perm_q),
                                             _p(d_y_perm_q_scales), _p(workspace), _nbytes(workspace), _stream()),
           "moe_grouped_mlp_backward_data")


def moe_grouped_mlp_backward_weights_workspace_bytes(L, capacity, H, F, dtype):
    return lib.moe_grouped_mlp_backward_weights_workspace_bytes(L, capacity, H, F, dtype)


def moe_grouped_mlp_backward_weights(x_perm, offsets, d_y_perm, data_workspace, dW1, dW2, workspace, H, F,
                                     dtype=BF16):
    _need(offsets, torch.int32, "offsets")
    _need(dW1, torch.float32, "dW1")
    _need(dW2, torch.float32, "dW2")
    L = offsets.shape[0] - 1
    cap = x_perm.shape[0]
    _check(lib.moe_grouped_mlp_backward_weights(L, H, F, cap, dtype, _p(x_perm), _p(offsets), _p(d_y_perm),
                                                _p(data_workspace), _nbytes(data_workspace), _p(dW1), _p(dW2),
                                                _p(workspace), _nbytes(workspace), _stream()),
           "moe_grouped_mlp_backward_weights")


def moe_mx_columns_grouped_max_blocks(L, capacity):
    return lib.moe_mx_columns_grouped_max_blocks(L, capacity)


def moe_mx_quantize_columns_grouped(x, offsets, pb, codes, scales):
    _need(offsets, torch.int32, "offsets")
    _need(pb, torch.int32, "pb")
    L = offsets.shape[0] - 1
    cap, C = x.shape
    _check(lib.moe_mx_quantize_columns_grouped(L, cap, C, _p(x), _p(offsets), _p(pb), _p(codes), _p(scales),
                                               _stream()), "moe_mx_quantize_columns_grouped")
