"""Pins for the oracle's production scheduler (the asynchronous variant of
Algorithm 1): the whole-walk optimum that sets the capacity, and the
capacity fill, against the pages' Theta(B) table, hand-worked stepped tables
and brute force over every length vector."""

import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import schedule as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_full_scan_on_the_pages_two_request_table():
    """The reading notes' two-request example: its Theta(B) table rises again
    after B = 4 (1.925 -> 1.975), and the notes state that B = 3 is the global
    maximum of the whole table, so the whole-walk optimum admits one slot."""
    with open(os.path.join(GOLD, "scheduler_two_requests.json")) as f:
        g = json.load(f)
    c = np.array(g["c"], dtype=np.float32)
    out = S.admit_full_scan(c, np.array(g["sps"]))
    assert out["A"] == 1
    assert out["ell"].tolist() == g["ell"]
    assert out["theta_best"] == pytest.approx(g["theta_best"], abs=1e-6)


def test_full_scan_passes_a_local_peak():
    """Worked by hand.  One request, c = (1, 1, 1), so tau = 1 + m exactly.
    SPS = (100, 60, 40, 40): Theta(m) = 100, 120, 120, 160.  The early stop
    admits one slot (120 > 100, then 120 is not above 120); the whole walk
    peaks at m = 3 behind the plateau."""
    c = np.ones((1, 3), dtype=np.float32)
    sps = np.array([100.0, 60.0, 40.0, 40.0])
    assert S.admit(c, sps)["A"] == 1
    out = S.admit_full_scan(c, sps)
    assert out["A"] == 3 and out["ell"].tolist() == [3]
    assert out["theta_best"] == 160.0


def test_full_scan_takes_the_smallest_m_on_ties():
    """SPS = (100, 60, 40, 30): Theta(m) = 100, 120, 120, 120 — three equal
    maxima; an equal Theta buys no more slots."""
    c = np.ones((1, 3), dtype=np.float32)
    out = S.admit_full_scan(c, np.array([100.0, 60.0, 40.0, 30.0]))
    assert out["A"] == 1 and out["ell"].tolist() == [1]
    assert out["theta_best"] == 120.0


def test_capacity_fill_by_hand():
    """c = (1, 1, 1), SPS = (100, 60, 40, 40): a capacity of two slots gives
    tau = 3 and Theta = 3 * 40; capacities past the pool admit all three."""
    c = np.ones((1, 3), dtype=np.float32)
    sps = np.array([100.0, 60.0, 40.0, 40.0])
    out = S.admit_capacity(c, sps, 2)
    assert out["A"] == 2 and out["ell"].tolist() == [2] and out["theta_best"] == 120.0
    assert S.admit_capacity(c, sps, 99)["ell"].tolist() == [3]
    assert S.admit_capacity(c, sps, 0)["ell"].tolist() == [0]
    assert S.admit_capacity(c, sps, -5)["A"] == 0


def _dyadic_instance(rng, R, gamma):
    """Confidences k/8: every survival is a dyadic rational with at most 3
    gamma <= 50 fractional bits, exact in float64 and in Q50, so brute force
    in Fractions and the Q50 walk see the same numbers.  A staircase table
    (plateaus, then cliffs) makes the whole walk and the early stop differ."""
    c = (rng.integers(1, 9, size=(R, gamma)) / 8.0).astype(np.float32)
    n = R * (1 + gamma)
    steps = np.where(rng.random(n) < 0.35, rng.uniform(0.2, 0.5, size=n), 0.0)
    steps[0] = 0.0
    sps = np.floor(1000.0 * np.cumprod(1.0 - steps))
    return c, sps


def _brute_max_tau(c, B):
    """max over every length vector with sum(1 + l_r) = B of
    tau = sum_r (1 + sum_{j <= l_r} prod_{i <= j} c_{r,i}), exactly."""
    R, gamma = c.shape
    prefix = []
    for r in range(R):
        s, acc, row = Fraction(1), Fraction(0), [Fraction(0)]
        for j in range(gamma):
            s *= Fraction(float(c[r, j]))
            acc += s
            row.append(acc)
        prefix.append(row)
    best = None
    for ell in itertools.product(range(gamma + 1), repeat=R):
        if sum(1 + e for e in ell) == B:
            tau = sum(1 + prefix[r][ell[r]] for r in range(R))
            best = tau if best is None or tau > best else best
    return best


@pytest.mark.parametrize("R,gamma", [(1, 5), (2, 3), (3, 2), (2, 4), (4, 2)])
def test_full_scan_is_the_brute_force_optimum_over_every_batch(R, gamma):
    rng = np.random.default_rng(31 * R + gamma)
    for _ in range(6):
        c, sps = _dyadic_instance(rng, R, gamma)
        theta = {B: _brute_max_tau(c, B) * Fraction(float(sps[B - 1])) for B in range(R, R * (1 + gamma) + 1)}
        top = max(theta.values())
        B_star = min(B for B, t in theta.items() if t == top)
        out = S.admit_full_scan(c, sps)
        assert out["A"] == B_star - R
        assert Fraction(out["tau_fx"], S.ONE) * Fraction(float(sps[B_star - 1])) == top
        assert int(out["ell"].sum()) == out["A"]


def test_staircases_trap_the_early_stop():
    """On stepped tables the early stop sometimes ends below the whole-walk
    optimum; wherever the two differ, the whole walk is strictly better."""
    rng = np.random.default_rng(2024)
    differs = 0
    for _ in range(300):
        R, gamma = int(rng.integers(1, 5)), int(rng.integers(2, 6))
        c, sps = _dyadic_instance(rng, R, gamma)
        early, full = S.admit(c, sps), S.admit_full_scan(c, sps)
        if early["A"] != full["A"]:
            differs += 1
            assert full["A"] > early["A"]
            assert Fraction(full["tau_fx"]) * Fraction(float(sps[R + full["A"] - 1])) > \
                Fraction(early["tau_fx"]) * Fraction(float(sps[R + early["A"] - 1]))
    assert differs >= 10


@pytest.mark.parametrize("R,gamma", [(1, 4), (2, 3), (3, 2)])
def test_capacity_fill_is_tau_optimal_at_every_capacity(R, gamma):
    rng = np.random.default_rng(77 + 10 * R + gamma)
    for _ in range(4):
        c, sps = _dyadic_instance(rng, R, gamma)
        for K in range(0, R * gamma + 1):
            out = S.admit_capacity(c, sps, K)
            assert out["A"] == K and int(out["ell"].sum()) == K
            assert Fraction(out["tau_fx"], S.ONE) == _brute_max_tau(c, R + K)


def test_full_scan_never_below_the_early_stop():
    rng = np.random.default_rng(5)
    for _ in range(40):
        R, gamma = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        c, sps = _dyadic_instance(rng, R, gamma)
        early, full = S.admit(c, sps), S.admit_full_scan(c, sps)
        assert Fraction(full["tau_fx"]) * Fraction(float(sps[R + full["A"] - 1])) >= \
            Fraction(early["tau_fx"]) * Fraction(float(sps[R + early["A"] - 1]))


def test_production_capacity_lags_two_rounds():
    """Non-anticipation through the lag: round t's capacity is fixed by round
    t - 2, so redrawing rounds t - 1 and t changes which slots fill it but not
    how many."""
    rng = np.random.default_rng(11)
    R, gamma = 3, 4
    sps = np.floor(1000.0 * np.cumprod(1.0 - np.where(rng.random(R * (1 + gamma)) < 0.4, 0.3, 0.0)))
    rounds = [rng.uniform(0.3, 1.0, size=(R, gamma)).astype(np.float32) for _ in range(6)]
    base = S.production_schedule(rounds, sps, K_init=2)
    assert [o["K"] for o in base[:2]] == [2, 2]
    for t in range(2, 6):
        assert base[t]["K"] == S.admit_full_scan(rounds[t - 2], sps)["A"]
        redrawn = list(rounds)
        redrawn[t] = rng.uniform(0.3, 1.0, size=(R, gamma)).astype(np.float32)
        redrawn[t - 1] = rng.uniform(0.3, 1.0, size=(R, gamma)).astype(np.float32)
        other = S.production_schedule(redrawn, sps, K_init=2)
        assert other[t]["K"] == base[t]["K"]
        assert other[t]["A"] == min(base[t]["K"], R * gamma)   # every slot is a candidate here
