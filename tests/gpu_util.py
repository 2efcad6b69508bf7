"""Helpers for the GPU parity tests: upload/download of exact values and the
tolerance measure (max error relative to the oracle's largest magnitude)."""
import numpy as np
import torch

from oracle import moe_oracle as O

DEV = "cuda"
TOL = {"f32": 1e-5, "bf16": 2e-2, "mxfp8": 3e-2, "mxfp4": 3e-2, "probs": 1e-5, "logits": 1e-5}


def rel_inf(got, want):
    """max |got - want| / max |want| (both float64 arrays); max |got| if want is all zero."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.abs(want).max() if want.size else 0.0
    num = np.abs(got - want).max() if want.size else 0.0
    return num / den if den > 0 else (np.abs(got).max() if got.size else 0.0)


def to_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return O.bits_to_bf16(t.contiguous().view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def bf16_from_f64(v: np.ndarray, device=DEV) -> torch.Tensor:
    """Exact bf16 tensor from float64 values that are already bf16 values."""
    bits = O.bf16_to_bits(v).view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(bits)).to(device).view(torch.bfloat16)


def bf16_from_bits(bits: np.ndarray, device=DEV) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits.astype(np.uint16).view(np.int16))).to(device).view(torch.bfloat16)


def np_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def say(*a):
    print(*a, flush=True)
