"""Pins for the oracle's scheduler (Algorithm 1) against the pages' worked
examples, the optimality lemmas (brute force) and special cases."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import schedule as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def theta_float(entry):
    B, tau_fx, theta = entry
    return float(theta / S.ONE)


def test_single_request_worked_example():
    g = gold("scheduler_single_request.json")
    c = np.array([g["c"]], dtype=np.float32)
    out = S.admit(c, np.array(g["sps"], dtype=np.float64))
    assert out["ell"].tolist() == [g["admit"]]
    a = S.survival(c)[0]
    np.testing.assert_allclose(a, g["survival_printed"], atol=0.5e-3 + 1e-9)
    # the walk stops at the fifth row, so the trace holds all five Theta values
    thetas = [theta_float(t) for t in out["trace"]]
    assert len(thetas) == 5
    np.testing.assert_allclose(thetas, g["theta_printed"], atol=0.05 + 1e-9)
    taus = [t[1] / S.ONE for t in out["trace"]]
    np.testing.assert_allclose(taus, g["expected_printed"], atol=1.5e-3)
    assert out["theta_best"] == pytest.approx(1212.746, abs=1e-2)


def test_two_request_worked_example():
    g = gold("scheduler_two_requests.json")
    c = np.array(g["c"], dtype=np.float32)
    sps = np.array(g["sps"])
    out = S.admit(c, sps)
    assert out["ell"].tolist() == g["ell"]
    assert out["A"] == 1
    assert out["theta_best"] == pytest.approx(g["theta_best"], abs=1e-6)
    order = [[r + 1, j + 1] for _, r, j in out["pool"]]
    assert order == g["order_1based"]
    curve = S.theta_curve(c, sps)
    assert [b for b, _, _ in curve] == g["curve_B"]
    np.testing.assert_allclose([t for _, t, _ in curve], g["curve_tau"], atol=1e-6)
    np.testing.assert_allclose([th for _, _, th in curve], g["curve_theta"], atol=1e-3)
    # B = 3 is also the global maximum of the curve (the pages' sanity check)
    assert max(range(len(curve)), key=lambda m: curve[m][2]) == 1


def test_three_request_worked_example():
    g = gold("scheduler_three_requests.json")
    c = np.array(g["c"], dtype=np.float32)
    sps = np.array(g["sps"])
    np.testing.assert_allclose(S.survival(c), g["survival_printed"], atol=0.5e-3 + 1e-9)
    out = S.admit(c, sps)
    assert [[r + 1, j + 1] for _, r, j in out["pool"]] == g["order_1based"]
    assert out["ell"].tolist() == g["ell"]
    walk = out["trace"]
    assert [t[0] for t in walk] == g["walk_B"]
    np.testing.assert_allclose([t[1] / S.ONE for t in walk], g["walk_tau"], atol=1e-3)
    np.testing.assert_allclose([theta_float(t) for t in walk], g["walk_theta"], atol=1e-3)
    curve = S.theta_curve(c, sps)
    np.testing.assert_allclose([curve[3][1], curve[4][1]], g["continued_tau"], atol=1e-3)
    np.testing.assert_allclose([curve[3][2], curve[4][2]], g["continued_theta"], atol=1e-3)
    assert out["theta_best"] == pytest.approx(g["theta_best"], abs=1e-3)


def test_appendix_a_eq9_stops_before_lookahead_gain():
    g = gold("appendix_a.json")["eq9"]
    for c2 in (0.9, 0.0, 0.5):
        c = np.array([[g["a1"], c2]], dtype=np.float32)
        out = S.admit(c, np.array(g["sps"]))
        assert out["ell"].tolist() == [g["ell"]]
        th = [theta_float(t) for t in out["trace"]]
        assert th[0] == pytest.approx(g["theta0"], abs=1e-6)
        assert th[1] == pytest.approx(g["theta1"], abs=1e-6)
    la = gold("appendix_a.json")["lookahead"]
    cA = np.array([[g["a1"], la["c2_if_A"]]], dtype=np.float32)
    cB = np.array([[g["a1"], la["c2_if_B"]]], dtype=np.float32)
    assert S.theta_curve(cA, np.array(g["sps"]))[2][2] == pytest.approx(la["theta2_if_A"], abs=1e-6)
    # with c2 = 0 the second slot has a = 0 and is not a candidate at all; its
    # Theta would be (1 + 0.8 + 0) * 0.45
    assert len(S.theta_curve(cB, np.array(g["sps"]))) == 2
    assert (1 + 0.8) * 0.45 == pytest.approx(la["theta2_if_B"])
    assert S.admit_lookahead(cA, np.array(g["sps"]))["ell"].tolist() == [2]
    assert S.admit_lookahead(cB, np.array(g["sps"]))["ell"].tolist() == [0]


def _random_instance(rng, R, gamma):
    c = rng.uniform(0.02, 0.999, size=(R, gamma)).astype(np.float32)
    n = R * (1 + gamma)
    steps = rng.uniform(0.0, 0.35, size=n)
    steps[0] = 0.0
    sps = 1000.0 * np.cumprod(1.0 - steps)
    return c, sps


@pytest.mark.parametrize("R,gamma", [(1, 6), (2, 3), (3, 3), (4, 2), (2, 5), (6, 2)])
def test_greedy_prefix_is_brute_force_optimum_at_every_batch(R, gamma):
    """Lemmas 1-2 and step 3: the greedy prefix reaches the best tau at every B."""
    rng = np.random.default_rng(1000 * R + gamma)
    for _ in range(4):
        c, sps = _random_instance(rng, R, gamma)
        curve = S.theta_curve(c, sps)
        assert len(curve) == R * gamma + 1
        for B, tau, _ in curve:
            best = S.brute_force_tau(c, B)
            assert abs(Fraction(tau) - best) < Fraction(1, 10 ** 9)


@pytest.mark.parametrize("seed", range(12))
def test_early_stop_equals_global_max_when_unimodal(seed):
    rng = np.random.default_rng(seed)
    R, gamma = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    c, sps = _random_instance(rng, R, gamma)
    curve = S.theta_curve(c, sps)
    th = [t for _, _, t in curve]
    peak = int(np.argmax(th))
    unimodal = all(th[i] < th[i + 1] for i in range(peak)) and \
        all(th[i] >= th[i + 1] for i in range(peak, len(th) - 1))
    out = S.admit(c, sps)
    if unimodal:
        assert out["A"] == peak
    # in every case the causal walk stops at the first non-increase
    first_drop = next((m for m in range(1, len(th)) if th[m] <= th[m - 1]), len(th))
    assert out["A"] == first_drop - 1


def test_prefix_closure_and_lengths_match_admitted_slots():
    rng = np.random.default_rng(7)
    for _ in range(20):
        R, gamma = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        c, sps = _random_instance(rng, R, gamma)
        c[rng.uniform(size=c.shape) < 0.2] = 1.0      # exact ties along prefixes
        out = S.admit(c, sps)
        admitted = out["pool"][:out["A"]]
        for r in range(R):
            js = sorted(j for _, rr, j in admitted if rr == r)
            assert js == list(range(len(js)))          # a prefix 0..l_r-1
            assert out["ell"][r] == len(js)
        assert out["ell"].sum() == out["A"]


def test_equal_theta_stops():
    # Theta(0) = 1 * 3 = 3, Theta(1) = 1.5 * 2 = 3: not an improvement
    out = S.admit(np.array([[0.5]], dtype=np.float32), np.array([3.0, 2.0]))
    assert out["ell"].tolist() == [0]
    out = S.admit(np.array([[0.5]], dtype=np.float32), np.array([3.0, 2.0 + 1e-12]))
    assert out["ell"].tolist() == [1]


def test_flat_table_admits_every_positive_slot_and_q50_cutoff():
    c = np.array([[2.0 ** -26, 2.0 ** -26, 0.5], [0.9, 0.8, 0.7]], dtype=np.float32)
    sps = np.full(8, 100.0)
    out = S.admit(c, sps)
    # a = 2^-26 > 0 is a candidate; a = 2^-52 quantises to 0 and is not
    assert out["ell"].tolist() == [1, 3]
    assert S.quantise(S.survival(c))[0] == [1 << 24, 0, 0]


def test_steep_table_admits_nothing():
    c = np.full((4, 3), 0.99, dtype=np.float32)
    sps = np.array([1000.0] * 4 + [1.0] * 12)
    out = S.admit(c, sps)
    assert out["ell"].tolist() == [0, 0, 0, 0]
    assert out["theta_best"] == 4 * 1000.0


def test_exact_and_plain_float_agree_without_near_ties():
    rng = np.random.default_rng(99)
    for _ in range(30):
        R, gamma = int(rng.integers(1, 12)), int(rng.integers(1, 10))
        c, sps = _random_instance(rng, R, gamma)
        a = S.admit(c, sps)
        b = S.admit_float(c, sps)
        assert a["ell"].tolist() == b["ell"].tolist()
        assert a["theta_best"] == pytest.approx(b["theta_best"], rel=1e-12)


def test_short_table_is_rejected():
    with pytest.raises(ValueError):
        S.admit(np.full((2, 3), 0.5, dtype=np.float32), np.ones(7))
