"""The skewed-routing bias constant against the oracle's router (CPU)."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import synthetic as S  # noqa: E402
import make_c4_bias as C4  # noqa: E402


def test_c4_constant_matches_calibration_record():
    with open(os.path.join(HERE, "golden", "c4_bias.json")) as f:
        rec = json.load(f)
    assert S.C4_BIAS_SCALE == rec["c"]
    assert abs(rec["share_top38"] - 0.5) <= 0.01


def test_c4_bias_gives_half_the_assignments_to_the_top_tenth():
    # recomputed with the oracle's router on the calibration batch
    s = C4.scores()
    share = C4.top_share(s, S.C4_BIAS_SCALE)
    assert abs(share - 0.5) <= 0.01, share
    # and the bias is a Zipf-shaped ranking: monotone in the seeded rank, mean zero
    b = S.skewed_bias(S.REAL, C4.PERM_SEED, S.C4_BIAS_SCALE).numpy().astype(np.float64)
    assert abs(b.mean()) < 1e-6
    assert len(np.unique(np.round(b, 9))) == S.REAL.n_routed
