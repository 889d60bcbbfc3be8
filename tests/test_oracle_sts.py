"""Pins for the oracle's sequential temperature scaling and calibration
metrics: a hand-computed ECE in both of its forms, bin edges, ROC-AUC
against scikit-learn (ties included) and its invariance to the temperature,
and recovery of a planted overconfidence factor."""

import numpy as np
import pytest
from sklearn.metrics import roc_auc_score

from oracle import sts as S


def test_ece_by_hand():
    """Two bins: {0.05, 0.15} with no positive, {0.55, 0.95} with two.
    Weighted form: 0.5 |0 - 0.1| + 0.5 |1 - 0.75| = 0.175."""
    p = np.array([0.05, 0.15, 0.55, 0.95], dtype=np.float32)
    y = np.array([0, 0, 1, 1])
    assert S.ece(p, y, 2) == pytest.approx(0.175, abs=1e-7)
    assert S.ece(p, y, 2) == pytest.approx(0.5 * abs(0 - 0.1) + 0.5 * abs(1 - 0.75), abs=1e-7)


def test_ece_bin_edges():
    # 0.5 opens the upper of two bins, 1.0 stays in the last bin
    assert S.ece(np.array([0.5, 1.0], dtype=np.float32), np.array([1, 1]), 2) == pytest.approx(0.25, abs=1e-12)
    assert S.ece(np.array([0.0], dtype=np.float32), np.array([0]), 15) == 0.0


def test_auc_matches_sklearn_with_ties():
    rng = np.random.default_rng(0)
    for _ in range(5):
        s = np.round(rng.normal(size=500), 1)          # many ties
        y = rng.random(500) < 0.4
        assert S.auc_pairs(s, y) == pytest.approx(roc_auc_score(y, s), abs=1e-12)
    assert np.isnan(S.auc_pairs(np.ones(3), np.array([True, True, True])))


def _rollouts(rng, N, gamma, beta):
    """True conditional acceptance q ~ Beta(6, 2); the head reports
    logit(q) * beta (beta > 1: overconfident); each rollout accepts position
    k with probability q_k until its first rejection."""
    q = rng.beta(6.0, 2.0, size=(N, gamma))
    z = (np.log(q / (1.0 - q)) * beta).astype(np.float32)
    acc = rng.random((N, gamma)) < q
    n_acc = np.where(acc.all(axis=1), gamma, np.argmin(acc, axis=1))
    return z, n_acc


GRID = np.exp(np.linspace(np.log(0.25), np.log(8.0), 61)).astype(np.float32)
GRID[24] = 1.0                                          # log-spaced, with T = 1 itself


@pytest.mark.parametrize("beta", [2.0, 1.0])
def test_recovers_a_planted_overconfidence(beta):
    rng = np.random.default_rng(5)
    z, n_acc = _rollouts(rng, 40000, 3, beta)
    out = S.sts_fit(z, n_acc, GRID, 15)
    # with the truth at T = beta, the first position's fit lands within a few grid steps
    step = np.log(GRID[1] / GRID[0])
    assert abs(np.log(out["T"][0] / beta)) <= 4 * step
    # T = 1 is on the grid, so the first position cannot end worse than raw
    # (later positions build on different chains and are not comparable)
    assert out["ece_after"][0] <= out["ece_before"][0] + 1e-12
    assert np.all(out["ece_after"] < 0.02)
    if beta > 1:
        assert np.all(out["ece_before"] > 0.05)


def test_auc_is_the_raw_separation_on_the_reached_rollouts():
    rng = np.random.default_rng(6)
    z, n_acc = _rollouts(rng, 5000, 3, 2.0)
    out = S.sts_fit(z, n_acc, GRID, 15)
    for k in range(3):
        reach = n_acc >= k
        lab = n_acc[reach] >= k + 1
        assert out["auc"][k] == pytest.approx(roc_auc_score(lab, z[reach, k]), abs=1e-12)
        # temperature scaling keeps the order
        assert S.auc_pairs(S.sigmoid32(z[reach, k] / out["T"][k]), lab) == pytest.approx(out["auc"][k], abs=2e-3)


def test_teacher_temperatures_are_used():
    rng = np.random.default_rng(7)
    z, n_acc = _rollouts(rng, 3000, 3, 2.0)
    own = S.sts_fit(z, n_acc, GRID, 15)
    forced = S.sts_fit(z, n_acc, GRID, 15, teacher_T=own["T"])
    np.testing.assert_array_equal(forced["T"], own["T"])
    np.testing.assert_allclose(forced["ece_grid"], own["ece_grid"], atol=0)
