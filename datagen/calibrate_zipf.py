"""Calibrate beta of the skewed workload's zipf router bias.

The workload description asks for a zipf(1.1) expert popularity added to
the router logits "so that about 10-20% of tokens overflow".  Adding log p_i
at full strength sends almost every token to expert 0, so the bias is
b_r[i] = beta * log p_i and beta is chosen by bisection so that, on the
seed-0 inputs, the CPU oracle's routing drops 15% of the tokens at capacity
factor 1.0.  Prints beta; the value is stored as datagen.ZIPF_BETA.

Run: python -m datagen.calibrate_zipf
"""
import numpy as np

import datagen
from oracle import moe as O


def drop_rate(cfg, beta):
    b_r = (beta * datagen.zipf_log_popularity(cfg["E"])).astype(np.float32)
    x64 = O.widen(cfg["x"], cfg["dtype"])
    z = O.router_logits(x64, cfg["W_r"], b_r)
    idx = O.top_k(z, cfg["k"])
    C = O.capacity(cfg["T"], cfg["E"], cfg["k"], cfg["cf"])
    _, drop, _ = O.assign_slots(idx, cfg["E"], C)
    return drop.mean()


def main(target=0.15):
    cfg = datagen.make("zipf_skew", seed=0, with_experts=False)
    lo, hi = 0.0, 1.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if drop_rate(cfg, mid) < target:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi), 5)
    print(f"beta = {beta}  drop rate = {drop_rate(cfg, beta):.4f}  (beta = 1: {drop_rate(cfg, 1.0):.4f})")


if __name__ == "__main__":
    main()
