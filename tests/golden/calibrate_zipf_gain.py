"""Find the gain of the DeepSeek-V3-like workload's Zipf(s=1.2) router bias.

Runs only the CPU oracle on the seeded inputs of that workload (T=8192,
H=7168, E=256, top-8, sigmoid scores): logits = x . W_r, keys = logits + bias
with b_e = -1.2 * gain * ln(rank_e).  Bisection finds the smallest gain (to
1e-3) at which at least 26 of the 256 experts (~10%) receive no route, and
prints it together with the load statistics.  The printed value is the
ZIPF_GAIN_CFG3 constant of workloads/configs.py.

    python tests/golden/calibrate_zipf_gain.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))
from oracle import moe_oracle as O  # noqa: E402
from workloads import get_config  # noqa: E402
from workloads.gen import make_tokens, make_router_inputs, zipf_bias, to_numpy_f64  # noqa: E402

TARGET_EMPTY = 26


def empty_experts(logits, cfg, gain):
    bias = zipf_bias(cfg, gain).numpy()
    ids, _ = O.route_topk(logits, cfg.K, cfg.score, bias)
    counts = np.bincount(ids.ravel().astype(np.int64), minlength=cfg.E)
    return int((counts == 0).sum()), counts


def main():
    cfg = get_config(3)
    x = to_numpy_f64(make_tokens(cfg))
    wr = to_numpy_f64(make_router_inputs(cfg, zipf_gain=0.0)["w_router"])
    logits = O.router_logits(x, wr)
    lo, hi = 0.0, 4.0
    assert empty_experts(logits, cfg, hi)[0] >= TARGET_EMPTY
    while hi - lo > 1e-3:
        mid = 0.5 * (lo + hi)
        if empty_experts(logits, cfg, mid)[0] >= TARGET_EMPTY:
            hi = mid
        else:
            lo = mid
    gain = float(np.ceil(hi * 1000.0) / 1000.0)
    n0, counts = empty_experts(logits, cfg, gain)
    print(f"gain={gain:.3f} empty={n0} max_load={counts.max()} "
          f"top5={sorted(counts.tolist())[-5:]}")


if __name__ == "__main__":
    main()
