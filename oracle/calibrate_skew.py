"""Calibrate the Zipf-shaped router bias of the skewed-routing workload (writes workloads/skew_beta.json).

Test/workload infrastructure: it draws the workload's x and W_g from the
seeded generator (CPU), computes router logits with the oracle, and bisects
beta in bias[e] = -beta * 1.2 * ln(e + 1) until expert 0 receives 3x its fair
share T*k/E of the (token, expert) pairs under the oracle's top-k.

READING: a pure Zipf(1.2) popularity over 64 experts would give expert 0
about 29% of all pairs (18.7x its share), more than distinct top-4 selection
allows and far from the stated ~3x; so the Zipf law shapes the bias and beta
sets the strength. The share is a law-of-large-numbers quantity at 131072
pairs, so the beta found on CPU draws gives about 3x on GPU draws of the same
distribution as well (the harness logs the realised share).

Usage: python -m oracle.calibrate_skew [--target 3.0]
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle.moe_oracle import route_logits, round_to_f32, select_topk  # noqa: E402
import workloads as W  # noqa: E402


def expert0_share(l0: np.ndarray, beta: float, k: int) -> float:
    E = l0.shape[1]
    bias = -beta * 1.2 * np.log(np.arange(E) + 1.0)
    bias32 = bias.astype(np.float32).astype(np.float64)     # the bias is stored as float32
    idx = select_topk(round_to_f32(l0 + bias32[None, :]), k)
    return float((idx == 0).sum()) / (idx.size / E)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--target", type=float, default=3.0)
    ap.add_argument("--out", default=os.path.join(ROOT, "workloads", "skew_beta.json"))
    args = ap.parse_args(argv)
    cfg = W.get_config("skew")
    inp = W.make_inputs(cfg.replace(bias="none"), "cpu", with_experts=False)
    l0 = route_logits(inp["x"], inp["w_gate"], None)
    lo, hi = 0.0, 2.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if expert0_share(l0, mid, cfg.top_k) < args.target:
            lo = mid
        else:
            hi = mid
    beta = 0.5 * (lo + hi)
    share = expert0_share(l0, beta, cfg.top_k)
    table = {"default": beta, f"{cfg.name}:T{cfg.T}:seed{cfg.seed}": beta,
             "_note": "beta for bias[e] = -beta*1.2*ln(e+1); expert-0 share / fair share = %.4f on the CPU draw" % share}
    with open(args.out, "w") as f:
        json.dump(table, f, indent=1)
    print(f"beta={beta:.6f} share={share:.4f}x -> {args.out}")


if __name__ == "__main__":
    main()
