"""Seeded tensor generators for the MoE workloads.

Every tensor comes from its own torch generator whose seed is derived with
numpy's SeedSequence from (config seed, tensor id[, expert]).  Token rows,
router weights, bias, logits and mask are always drawn on the CPU, so they are
identical on every machine with this software stack.  Expert weights are
drawn per expert on the device that asks for them (the CPU generator and the
GPU generator give different, equally valid streams); a test that checks the
GPU against the oracle hands the oracle a host copy of the very tensors the
GPU used.

Values are drawn in fp32 ~ N(0, std) and rounded to bf16 by torch's
round-to-nearest-even cast where the workload is bf16.
"""
import math

import numpy as np
import torch

from .configs import MoEConfig, ZIPF_GAIN_CFG3, GROUP_OFFSET_CFG5

# tensor ids for seed derivation
_TID_X, _TID_WR, _TID_W1, _TID_W2, _TID_BIAS, _TID_LOGITS, _TID_GROUPS = range(1, 8)


def _seed(cfg_seed: int, tid: int, e: int = 0) -> int:
    ss = np.random.SeedSequence([int(cfg_seed), int(tid), int(e)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, seed, device="cpu", dtype=torch.float32):
    g = _gen(seed, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def _tdtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16, "mxfp8": torch.bfloat16, "mxfp4": torch.bfloat16}[name]


def make_tokens(cfg: MoEConfig, T: int = None, seed: int = None) -> torch.Tensor:
    """x [T,H] on the CPU in the workload's activation dtype."""
    T = cfg.T if T is None else T
    s = cfg.seed if seed is None else seed
    return _normal((T, cfg.H), cfg.x_std, _seed(s, _TID_X), dtype=_tdtype(cfg.x_dtype))


def zipf_bias(cfg: MoEConfig, gain: float, seed: int = None) -> torch.Tensor:
    """Per-expert additive router bias with Zipf(s=1.2) selection odds.

    A seeded permutation gives each expert a popularity rank r_e in 1..E and
    b_e = -1.2 * gain * ln(r_e), so exp(b_e) ~ r_e^(-1.2 gain).
    """
    s = cfg.seed if seed is None else seed
    g = _gen(_seed(s, _TID_BIAS))
    ranks = torch.randperm(cfg.E, generator=g).to(torch.float64) + 1.0
    return (-1.2 * gain * torch.log(ranks)).to(torch.float32)


def grouped_logits(cfg: MoEConfig, T: int = None, seed: int = None) -> torch.Tensor:
    """Router logits [T,E] fp32 for the large-top-K share.

    z ~ N(0,1); experts come in groups of 32 (group g = ids 32g..32g+31, group
    0 = the local experts).  Each token draws group 0 plus 7 distinct groups
    out of the remaining ones and gets GROUP_OFFSET_CFG5 added to those 8
    groups' logits, so its top-36 lies in the drawn groups and each drawn group
    receives 4.5 routes on average.
    """
    T = cfg.T if T is None else T
    s = cfg.seed if seed is None else seed
    z = _normal((T, cfg.E), 1.0, _seed(s, _TID_LOGITS))
    ngroups = cfg.E // 32
    g = _gen(_seed(s, _TID_GROUPS))
    pick = torch.rand((T, ngroups - 1), generator=g).argsort(dim=1)[:, :7] + 1
    chosen = torch.zeros((T, ngroups), dtype=torch.bool)
    chosen[:, 0] = True
    chosen.scatter_(1, pick, True)
    offs = chosen.repeat_interleave(32, dim=1).to(torch.float32) * GROUP_OFFSET_CFG5
    return (z + offs).contiguous()


def make_router_inputs(cfg: MoEConfig, T: int = None, seed: int = None, zipf_gain: float = None):
    """Router-side inputs on the CPU.

    Returns a dict with
      'w_router' [H,E] (fp32 or bf16) or None when logits are given,
      'bias' [E] fp32 or None, 'logits' [T,E] fp32 or None,
      'mask' [T] uint8 (1 = masked token) or None.
    """
    T = cfg.T if T is None else T
    s = cfg.seed if seed is None else seed
    out = {"w_router": None, "bias": None, "logits": None, "mask": None}
    if cfg.logits == "proj":
        out["w_router"] = _normal((cfg.H, cfg.E), cfg.w_std, _seed(s, _TID_WR),
                                  dtype=_tdtype(cfg.wr_dtype))
    else:
        out["logits"] = grouped_logits(cfg, T, s)
    if cfg.bias == "zipf":
        out["bias"] = zipf_bias(cfg, ZIPF_GAIN_CFG3 if zipf_gain is None else zipf_gain, s)
    if cfg.mask_every:
        t = torch.arange(T)
        out["mask"] = (t % cfg.mask_every == cfg.mask_every - 1).to(torch.uint8)
    return out


def make_expert_weights(cfg: MoEConfig, e: int, device="cpu", seed: int = None):
    """Logical expert weights (W1[e] [H,2F], W2[e] [F,H]) drawn on `device`.

    Gate columns of W1 are [0,F), up columns [F,2F).  bf16 for the bf16 and
    MXFP8 workloads (MX quantization is part of the layer), fp32 otherwise.
    """
    s = cfg.seed if seed is None else seed
    dt = _tdtype(cfg.dtype)
    w1 = _normal((cfg.H, 2 * cfg.F), cfg.w_std, _seed(s, _TID_W1, e), device, dt)
    w2 = _normal((cfg.F, cfg.H), cfg.w_std, _seed(s, _TID_W2, e), device, dt)
    return w1, w2


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16 tensor (as a numpy array on the host)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_float(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_numpy_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a CPU/GPU tensor of dtype fp32 or bf16."""
    if t.dtype == torch.bfloat16:
        return bits_to_float(bf16_bits(t))
    return t.detach().cpu().numpy().astype(np.float64)


def approx_gb(nbytes: int) -> str:
    return f"{nbytes / 1e9:.2f} GB" if nbytes >= 1e8 else f"{nbytes / 1e6:.2f} MB"


__all__ = ["make_tokens", "make_router_inputs", "make_expert_weights", "zipf_bias",
           "grouped_logits", "bf16_bits", "bits_to_float", "to_numpy_f64", "math"]
