#!/usr/bin/env python3
"""Calibrate the skewed-routing bias of the 2048-token prefill with slots.

The bias is b_e = -c * 1.1 * ln(rank_e) over a seeded permutation of the
ranks 1..384, mean removed (a Zipf(1.1)-shaped preference). c is found by
bisection with the oracle's router on a separate calibration batch of 2048
tokens so that the 38 most loaded experts (10%) take 50% of the 12,288
assignments. Writes c4_bias.json next to this file; the constant
synthetic.gen.C4_BIAS_SCALE must carry the same value.

Only the seeded input generators and oracle/ are used.
"""
import json
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synthetic as S  # noqa: E402

LAYER_SEED = 1          # the real layer's router
PERM_SEED = 4           # the skewed configuration's rank permutation
CALIB_INDEX = 1         # calibration tokens: seed 4, batch 1 (the benchmark uses batch 0)
M = 2048
TOP = 38
TARGET = 0.50


def bits(t):
    return t.detach().contiguous().view(torch.int16).numpy().view(np.uint16)


def scores():
    shape = S.REAL
    wr, _ = S.make_router(shape, LAYER_SEED, 0.02, None)
    x = S.make_tokens(M, shape.dim, PERM_SEED, index=CALIB_INDEX)
    z = oracle.router_logits(oracle.bf16_bits_to_f64(bits(x)), oracle.bf16_bits_to_f64(bits(wr)))
    return oracle.sqrt_softplus_scores(z, 1.0)


def top_share(s, c):
    """Share of the assignments taken by the TOP most loaded experts under bias scale c."""
    bias = S.skewed_bias(S.REAL, PERM_SEED, c).numpy().astype(np.float64)
    idx = oracle.select_topk(s + bias[None, :], S.REAL.topk)
    counts = np.bincount(idx.reshape(-1), minlength=S.REAL.n_routed)
    return float(np.sort(counts)[::-1][:TOP].sum() / counts.sum())


def main():
    s = scores()
    lo, hi = 0.0, 1.0
    while top_share(s, hi) < TARGET:
        hi *= 2.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if top_share(s, mid) < TARGET:
            lo = mid
        else:
            hi = mid
    c = round(hi, 6)
    share = top_share(s, c)
    rec = {"c": c, "share_top38": share, "tokens": M, "assignments": M * S.REAL.topk, "layer_seed": LAYER_SEED,
           "perm_seed": PERM_SEED, "calibration_batch": CALIB_INDEX}
    with open(os.path.join(HERE, "c4_bias.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
