"""Pins for the oracle's two further verification modes: greedy
(temperature-0) exact-match verification and the analytic acceptance
c*_k = sum_v min(p_d, p_t), against the pages' worked example, eq (8c),
the rejection-sampling rate it stands for, special cases, and the
temperature-to-zero limit of stochastic verification."""

import json
import os

import numpy as np
import pytest

from oracle import verify as Vf

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _instance(rng, R, gamma, V, r, scale=1.0):
    U = rng.normal(0.0, 2.0, size=(R, gamma, V))
    E = rng.normal(0.0, 0.5, size=(V, r))
    W2t = rng.normal(0.0, 0.5, size=(V, r))
    x0 = rng.integers(0, V, size=R)
    x = rng.integers(0, V, size=(R, gamma))
    target = rng.normal(0.0, 2.0 * scale, size=(R, gamma + 1, V))
    return target, U, E, W2t, x0, x


def _softmax(l):
    e = np.exp(l - l.max())
    return e / e.sum()


def test_analytic_acceptance_page_example():
    """The notes' check of eq (8a)-(8c): p_t = (0.7, 0.3), p_d = (0.5, 0.5)."""
    g = json.load(open(os.path.join(GOLD, "acceptance_identity.json")))
    target = np.log(np.array(g["p_t"]))[None, None, :]
    U = np.log(np.array(g["p_d"]))[None, None, :]
    E = np.zeros((2, 4))
    out = Vf.analytic_acceptance(target, None, U, E, E, np.array([0]), np.array([[1]]))
    assert out[0, 0] == pytest.approx(g["sum_min"], abs=1e-12)
    assert out[0, 0] == pytest.approx(1.0 - 0.5 * g["l1"], abs=1e-12)


def test_analytic_acceptance_is_one_minus_half_l1():
    """eq (8c), with p_d built here from U_k + W1[x_{k-1}] W2 directly."""
    rng = np.random.default_rng(3)
    target, U, E, W2t, x0, x = _instance(rng, 3, 4, 50, 8)
    c = Vf.analytic_acceptance(target, None, U, E, W2t, x0, x)
    for r in range(3):
        for k in range(4):
            prev = x0[r] if k == 0 else x[r, k - 1]
            pd = _softmax(U[r, k] + W2t @ E[prev])
            pt = _softmax(target[r, k])
            assert c[r, k] == pytest.approx(1.0 - 0.5 * np.abs(pd - pt).sum(), abs=1e-12)


def test_analytic_acceptance_is_the_rejection_sampling_rate():
    """Drafting x ~ p_d and running the oracle's stochastic accept test
    accepts with probability c* (the quantity eq (8a) marginalises)."""
    rng = np.random.default_rng(8)
    V = 12
    target, U, E, W2t, x0, _ = _instance(rng, 1, 1, V, 4)
    ld = U[0, 0] + W2t @ E[x0[0]]
    pd = _softmax(ld)
    c = Vf.analytic_acceptance(target, None, U, E, W2t, x0, np.zeros((1, 1), dtype=np.int64))[0, 0]
    n = 40000
    xs = rng.choice(V, size=n, p=pd)
    u = rng.random(n)
    acc = 0
    for xi, ui in zip(xs, u):
        lr = Vf.accept_log_ratios(target, None, U, E, W2t, x0, np.array([[xi]]), np.array([1]))[0]
        acc += Vf.first_rejection(lr, np.array([ui])) == 1
    sd = np.sqrt(c * (1 - c) / n)
    assert abs(acc / n - c) < 5 * sd


def test_analytic_acceptance_special_cases():
    V = 6
    E = np.zeros((V, 2))
    l = np.array([0.3, -1.0, 2.0, 0.0, 0.5, -0.2])
    same = Vf.analytic_acceptance((l + 7.0)[None, None, :], None, l[None, None, :], E, E,
                                  np.array([0]), np.array([[0]]))
    assert same[0, 0] == pytest.approx(1.0, abs=1e-12)       # identical distributions
    t = np.array([0.0, 0.0, 0.0, -np.inf, -np.inf, -np.inf])
    d = np.array([-np.inf, -np.inf, -np.inf, 0.0, 0.0, 0.0])
    apart = Vf.analytic_acceptance(t[None, None, :], None, d[None, None, :], E, E,
                                   np.array([0]), np.array([[0]]))
    assert apart[0, 0] == 0.0                                   # disjoint supports


def test_analytic_acceptance_takes_the_given_normaliser():
    rng = np.random.default_rng(4)
    target, U, E, W2t, x0, x = _instance(rng, 2, 3, 30, 4)
    own = Vf.analytic_acceptance(target, None, U, E, W2t, x0, x)
    lse = np.array([[np.log(np.exp(Vf.draft_logits_at(U, E, W2t, x0, x, r, k)).sum()) for k in range(3)]
                    for r in range(2)])
    np.testing.assert_allclose(Vf.analytic_acceptance(target, None, U, E, W2t, x0, x, lse), own, atol=1e-12)
    # a normaliser larger by ln 2 halves p_d
    shifted = Vf.analytic_acceptance(target, None, U, E, W2t, x0, x, lse + np.log(2.0))
    r, k = 1, 2
    pd = _softmax(Vf.draft_logits_at(U, E, W2t, x0, x, r, k)) / 2.0
    assert shifted[r, k] == pytest.approx(np.minimum(pd, _softmax(target[r, k])).sum(), abs=1e-12)


def test_greedy_by_hand():
    """Rows' argmaxes are 2, 0, 3, 1; drafts (2, 0, 1): the third mismatches."""
    target = np.array([[[0, 1, 5, 2], [9, 1, 5, 2], [0, 1, 2, 3], [0, 4, 2, 3]]], dtype=np.float64)
    out = Vf.verify_greedy(target, None, np.array([[2, 0, 1]]), np.array([3]))
    assert out["n_acc"].tolist() == [2] and out["next_tok"].tolist() == [3]
    out = Vf.verify_greedy(target, None, np.array([[2, 0, 3]]), np.array([3]))
    assert out["n_acc"].tolist() == [3] and out["next_tok"].tolist() == [1]   # bonus row
    out = Vf.verify_greedy(target, None, np.array([[2, 0, 3]]), np.array([0]))
    assert out["n_acc"].tolist() == [0] and out["next_tok"].tolist() == [2]   # nothing admitted


def test_greedy_ties_take_the_lowest_index():
    target = np.array([[[3.0, 5.0, 5.0, 1.0], [2.0, 2.0, 2.0, 2.0]]])
    out = Vf.verify_greedy(target, None, np.array([[2]]), np.array([1]))
    assert out["n_acc"].tolist() == [0] and out["next_tok"].tolist() == [1]
    out = Vf.verify_greedy(target, None, np.array([[1]]), np.array([1]))
    assert out["n_acc"].tolist() == [1] and out["next_tok"].tolist() == [0]


@pytest.mark.parametrize("seed", range(6))
def test_greedy_is_the_zero_temperature_limit(seed):
    """Target logits scaled by 1/T, T -> 0 (distinct integer logits keep the
    argmax gap at 1/T): stochastic verification accepts exactly the drafts
    that equal the argmax and draws the argmax next."""
    rng = np.random.default_rng(seed)
    R, gamma, V, r = 4, 5, 20, 4
    _, U, E, W2t, x0, _ = _instance(rng, R, gamma, V, r)
    target = np.stack([[rng.permutation(V).astype(np.float64) for _ in range(gamma + 1)] for _ in range(R)])
    am = target.argmax(axis=2)
    # drafts that follow the argmax for a random number of positions
    x = rng.integers(0, V, size=(R, gamma))
    for q in range(R):
        keep = int(rng.integers(0, gamma + 1))
        x[q, :keep] = am[q, :keep]
    ell = rng.integers(0, gamma + 1, size=R)
    greedy = Vf.verify_greedy(target, None, x, ell)
    cold = Vf.verify(target / 1e-3, None, U, E, W2t, x0, x, ell,
                     rng.uniform(1e-6, 1.0, size=(R, gamma)), rng.uniform(0.0, 1.0, size=R))
    assert greedy["n_acc"].tolist() == cold["n_acc"].tolist()
    assert greedy["next_tok"].tolist() == cold["next_tok"].tolist()
