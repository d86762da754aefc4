"""Pins for the oracle's routing: scores, the biased stable top-k and the weights.

Independent checks: closed forms of the thresholded softplus, a brute-force
rank formulation of the selection (rank_e = number of experts that beat e),
constructed ties, NaN handling, and the normalisation invariant.
"""
import math

import numpy as np
import pytest

from oracle import moe_ref as R


def test_softplus_closed_forms():
    assert R.softplus_thresholded(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    a = 1.0
    assert R.softplus_thresholded(math.log(math.e - 1.0)) == pytest.approx(a, rel=1e-15)
    assert R.softplus_thresholded(25.0) == 25.0            # above the threshold: identity
    assert R.softplus_thresholded(20.0) > 20.0             # at 20 the log branch is taken
    assert R.softplus_thresholded(20.0) - 20.0 == pytest.approx(math.exp(-20.0), rel=1e-6)
    assert R.softplus_thresholded(-30.0) == pytest.approx(math.exp(-30.0), rel=1e-12)


def test_scores_temperature_and_sqrt():
    z = np.array([[0.0, 50.0, 2.0 * math.log(math.e ** 4 - 1.0)]])
    s = R.sqrt_softplus_scores(z, gate_temp=2.0)
    assert s[0, 0] == pytest.approx(math.sqrt(math.log(2.0)), rel=1e-15)
    assert s[0, 1] == pytest.approx(5.0, rel=1e-15)         # 50/2 = 25 > 20 -> sqrt(25)
    assert s[0, 2] == pytest.approx(2.0, rel=1e-14)         # softplus(ln(e^4 - 1)) = 4


def brute_force_topk(keys, k):
    """rank_e = #{e' : key_e' > key_e, or key_e' == key_e and e' < e}; picks are the
    experts of rank < k, listed by rank."""
    n = len(keys)
    rank = [sum(1 for f in range(n) if keys[f] > keys[e] or (keys[f] == keys[e] and f < e)) for e in range(n)]
    return [rank.index(r) for r in range(k)]


@pytest.mark.parametrize("seed", range(30))
def test_topk_against_rank_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 12))
    k = int(rng.integers(1, n + 1))
    keys = rng.integers(-3, 4, size=(5, n)).astype(np.float64) * 0.25   # many ties
    got = R.select_topk(keys, k)
    for t in range(5):
        assert list(got[t]) == brute_force_topk(list(keys[t]), k)


def test_topk_all_equal_picks_lowest_ids():
    keys = np.full((3, 16), 0.7)
    assert np.array_equal(R.select_topk(keys, 4), np.tile(np.arange(4), (3, 1)))


def test_topk_nan_is_an_error():
    keys = np.array([[0.1, np.nan, 0.3]])
    with pytest.raises(R.NonFiniteKey):
        R.select_topk(keys, 2)


def test_weights_sum_to_route_scale():
    cfg = R.MoeCfg(dim=256, inter=256, n_routed=16, topk=4, route_scale=1.5)
    rng = np.random.default_rng(3)
    s = rng.uniform(0.1, 3.0, size=(50, 4))
    g = R.routing_weights(s, cfg)
    assert np.all(np.abs(g.sum(axis=1) - 1.5) <= 4 * np.finfo(np.float64).eps)
    # proportional to the scores
    assert np.allclose(g / s, (g / s)[:, :1])


def test_weights_k1_and_norm_off_skip_normalisation():
    s = np.array([[0.8], [2.0]])
    cfg1 = R.MoeCfg(dim=256, inter=256, n_routed=16, topk=1, route_scale=1.5)
    assert np.array_equal(R.routing_weights(s, cfg1), 1.5 * s)
    s2 = np.array([[0.5, 0.25]])
    cfg2 = R.MoeCfg(dim=256, inter=256, n_routed=16, topk=2, route_scale=2.0, norm_topk_prob=False)
    assert np.array_equal(R.routing_weights(s2, cfg2), 2.0 * s2)


def test_route_bias_steers_selection_not_weights():
    cfg = R.MoeCfg(dim=4, inter=256, n_routed=3, topk=1, route_scale=1.0)
    x = np.array([[1.0, 0.0, 0.0, 0.0]])
    wr = np.array([[3.0, 0, 0, 0], [1.0, 0, 0, 0], [0.0, 0, 0, 0]])
    bias = np.array([0.0, 10.0, 0.0])
    idx, g, keys, s = R.route(cfg, x, wr, bias)
    assert idx[0, 0] == 1                       # the bias wins the selection
    assert g[0, 0] == pytest.approx(math.sqrt(math.log1p(math.e)), rel=1e-15)   # weight: unbiased s_1


def test_route_threshold_branch_reached():
    cfg = R.MoeCfg(dim=2, inter=256, n_routed=2, topk=1, route_scale=1.0)
    x = np.array([[1.0, 1.0]])
    wr = np.array([[20.0, 16.0], [0.0, 0.0]])   # z = 36 > 20 -> s = 6 exactly
    idx, g, keys, s = R.route(cfg, x, wr, np.zeros(2))
    assert s[0, 0] == 6.0 and idx[0, 0] == 0 and g[0, 0] == 6.0
