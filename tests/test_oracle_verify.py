"""Pins for the oracle's verifier: the acceptance identity eq (8a)-(8c), the
lossless property (the emitted token is distributed as p_t), Appendix A's
eq (10), and indexing special cases.

Distributions are measured without randomness where possible: the accept
decision and the inverse-CDF draw are step functions of their uniform, so
evaluating them on a midpoint grid of N uniforms measures each probability to
within 1/N."""

import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import schedule as S
from oracle import verify as Vf
from oracle.sample import markov_sample

GOLD = os.path.join(os.path.dirname(__file__), "golden")
N_GRID = 2000


def grid(n=N_GRID):
    return (np.arange(n) + 0.5) / n


def one_position_instance(p_t, p_d):
    """R=1, gamma=1: U carries log p_d (bias zero: W1 = W2 = 0), target row 0
    carries log p_t, row 1 is an unrelated bonus row."""
    V = len(p_t)
    U = np.log(np.asarray(p_d, dtype=np.float64))[None, None, :]
    tgt = np.zeros((1, 2, V))
    tgt[0, 0] = np.log(np.asarray(p_t, dtype=np.float64))
    tgt[0, 1] = np.linspace(0.0, 1.0, V)
    E = np.zeros((V, 4))
    W2t = np.zeros((V, 4))
    return U, tgt, E, W2t


def accept_fraction(U, tgt, E, W2t, x_tok):
    """Fraction of a uniform grid for which draft token x_tok is accepted."""
    x0 = np.array([0])
    x = np.array([[x_tok]])
    logr = Vf.accept_log_ratios(tgt, None, U, E, W2t, x0, x, np.array([1]))[0]
    return float(np.mean([Vf.first_rejection(logr, np.array([u])) == 1 for u in grid()]))


def residual_distribution(U, tgt, E, W2t, x_tok):
    """Distribution of the resampled token after a rejection of x_tok."""
    V = U.shape[2]
    x0 = np.array([0])
    x = np.array([[x_tok]])
    res = Vf.residual(tgt, None, U, E, W2t, x0, x, 0, 0, 1)
    counts = np.zeros(V)
    for u in grid():
        counts[Vf.inverse_cdf(res, u)] += 1
    return counts / N_GRID


def emitted_distribution(p_t, p_d):
    """P(first emitted token = y) for one drafted position, enumerating the
    draft x ~ p_d exactly and the two uniforms on grids."""
    U, tgt, E, W2t = one_position_instance(p_t, p_d)
    V = len(p_t)
    out = np.zeros(V)
    acc_total = 0.0
    for xt in range(V):
        pa = accept_fraction(U, tgt, E, W2t, xt)
        acc_total += p_d[xt] * pa
        out[xt] += p_d[xt] * pa
        if pa < 1.0:
            out += p_d[xt] * (1.0 - pa) * residual_distribution(U, tgt, E, W2t, xt)
    return out, acc_total


def test_acceptance_identity_worked_example():
    g = json.load(open(os.path.join(GOLD, "acceptance_identity.json")))
    p_t, p_d = np.array(g["p_t"]), np.array(g["p_d"])
    assert np.minimum(p_t, p_d).sum() == pytest.approx(g["sum_min"])
    assert np.abs(p_t - p_d).sum() == pytest.approx(g["l1"])
    _, acc = emitted_distribution(p_t, p_d)
    assert acc == pytest.approx(g["accept_prob"], abs=1.0 / N_GRID)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_lossless_and_acceptance_rate_by_grid(seed):
    rng = np.random.default_rng(seed)
    V = 5
    p_t = rng.dirichlet(np.ones(V))
    p_d = rng.dirichlet(np.ones(V))
    dist, acc = emitted_distribution(p_t, p_d)
    # invariant (a): the emitted token is distributed as p_t
    np.testing.assert_allclose(dist, p_t, atol=3.0 / N_GRID)
    # invariant (b): acceptance probability = 1 - TV(p_d, p_t)
    assert acc == pytest.approx(1.0 - 0.5 * np.abs(p_d - p_t).sum(), abs=1.0 / N_GRID)


def test_lossless_chi_square_with_sampled_drafts():
    """End to end with seeded draws: drafts from the oracle sampler, then the
    verifier; the first emitted token must follow p_t (chi-square)."""
    rng = np.random.default_rng(2026)
    V, R = 6, 20000
    p_t = np.array([0.30, 0.05, 0.25, 0.10, 0.20, 0.10])
    p_d = np.array([0.10, 0.30, 0.15, 0.25, 0.05, 0.15])
    U = np.broadcast_to(np.log(p_d), (R, 1, V)).copy()
    E = np.zeros((V, 4))
    W2t = np.zeros((V, 4))
    x0 = np.zeros(R, dtype=np.int64)
    G = -np.log(-np.log(rng.uniform(size=(R, 1, 1))))
    g = -np.log(-np.log(rng.uniform(size=(R, 1, 64))))
    x = markov_sample(U, E, W2t, x0, G, g)["x"]
    tgt = np.zeros((R, 2, V))
    tgt[:, 0, :] = np.log(p_t)
    tgt[:, 1, :] = 0.0
    out = Vf.verify(tgt, None, U, E, W2t, x0, x, np.ones(R, dtype=np.int64),
                    rng.uniform(size=(R, 1)), rng.uniform(size=R))
    first = np.where(out["n_acc"] == 1, x[:, 0], out["next_tok"])
    counts = np.bincount(first, minlength=V)
    p = stats.chisquare(counts, R * p_t).pvalue
    assert p > 1e-3
    acc_rate = out["n_acc"].mean()
    z = (acc_rate - np.minimum(p_t, p_d).sum()) / np.sqrt(0.25 / R)
    assert abs(z) < 4.0


def test_appendix_a_eq10_lookahead_biases_the_output():
    g = json.load(open(os.path.join(GOLD, "appendix_a.json")))
    p_t, p_d = np.array(g["eq10"]["p_t"]), np.array(g["eq10"]["p_d"])
    sps = np.array(g["eq9"]["sps"])
    a1 = g["eq9"]["a1"]
    c2 = {0: g["lookahead"]["c2_if_A"], 1: g["lookahead"]["c2_if_B"]}
    # gamma = 2; both target rows carry p_t, the draft carries p_d at both positions
    U = np.log(np.broadcast_to(p_d, (1, 2, 2))).copy()
    tgt = np.log(np.broadcast_to(p_t, (1, 3, 2))).copy()
    E = np.zeros((2, 4))
    W2t = np.zeros((2, 4))
    x0 = np.array([0])

    def pr_first_is_A(scheduler):
        total = 0.0
        for x1 in (0, 1):
            c = np.array([[a1, c2[x1]]], dtype=np.float32)
            ell = scheduler(c, sps)["ell"]
            x = np.array([[x1, 0]])
            logr = Vf.accept_log_ratios(tgt, None, U, E, W2t, x0, x, ell)[0]
            pa = 0.0
            for u in grid():
                n = Vf.first_rejection(logr, np.array([u, 0.5]))
                if n >= 1:
                    pa += (x1 == 0)
                else:
                    res = Vf.residual(tgt, None, U, E, W2t, x0, x, 0, 0, int(ell[0]))
                    pa += np.mean([Vf.inverse_cdf(res, v) == 0 for v in grid(200)])
            total += p_d[x1] * pa / N_GRID
        return total

    assert pr_first_is_A(S.admit) == pytest.approx(g["eq10"]["pr_A_causal"], abs=5e-3)
    assert pr_first_is_A(S.admit_lookahead) == pytest.approx(g["eq10"]["pr_A_lookahead"], abs=5e-3)


def _instance(rng, R=3, gamma=4, V=40, r=8):
    U = rng.normal(0, 2, size=(R, gamma, V))
    E = rng.normal(0, 0.3, size=(V, r))
    W2t = rng.normal(0, 0.3, size=(V, r))
    x0 = rng.integers(0, V, size=R)
    x = rng.integers(0, V, size=(R, gamma))
    return U, E, W2t, x0, x


def _draft_logits(U, E, W2t, x0, x):
    R, gamma, V = U.shape
    L = np.zeros_like(U)
    for r in range(R):
        for i in range(gamma):
            L[r, i] = Vf.draft_logits_at(U, E, W2t, x0, x, r, i)
    return L


def test_all_accepted_draws_the_bonus_row():
    rng = np.random.default_rng(5)
    U, E, W2t, x0, x = _instance(rng)
    R, gamma, V = U.shape
    tgt = np.zeros((R, gamma + 1, V))
    tgt[:, :gamma] = _draft_logits(U, E, W2t, x0, x)    # p_t == p_d: ratio 1
    ell = np.array([4, 2, 0])
    bonus = np.array([7, 11, 3])
    for r in range(R):
        tgt[r, ell[r], :] = -60.0
        tgt[r, ell[r], bonus[r]] = 0.0                  # bonus row ~ one-hot
    out = Vf.verify(tgt, None, U, E, W2t, x0, x, ell,
                    np.full((R, gamma), 1.0 - 2.0 ** -24), np.full(R, 0.5))
    assert out["n_acc"].tolist() == ell.tolist()
    assert out["next_tok"].tolist() == bonus.tolist()


def test_first_rejection_position_and_residual_excludes_rejected_token():
    rng = np.random.default_rng(6)
    U, E, W2t, x0, x = _instance(rng, R=1)
    R, gamma, V = U.shape
    tgt = np.zeros((R, gamma + 1, V))
    tgt[:, :gamma] = _draft_logits(U, E, W2t, x0, x)
    tgt[0, 2, x[0, 2]] = -80.0                          # p_t(x_2) ~ 0 at row 2 only
    out = Vf.verify(tgt, None, U, E, W2t, x0, x, np.array([4]),
                    np.full((1, gamma), 0.5), np.array([0.5]))
    assert out["n_acc"].tolist() == [2]
    assert out["next_tok"][0] != x[0, 2]
    res = Vf.residual(tgt, None, U, E, W2t, x0, x, 0, 2, 4)
    assert res[x[0, 2]] == 0.0


def test_packed_rows_match_dense_layout():
    rng = np.random.default_rng(8)
    U, E, W2t, x0, x = _instance(rng)
    R, gamma, V = U.shape
    tgt = rng.normal(0, 2, size=(R, gamma + 1, V))
    ell = np.array([2, 0, 4])
    u_acc = rng.uniform(size=(R, gamma))
    u_res = rng.uniform(size=R)
    dense = Vf.verify(tgt, None, U, E, W2t, x0, x, ell, u_acc, u_res)
    rows, row0 = [], []
    for r in range(R):
        row0.append(len(rows))
        rows.extend(tgt[r, :ell[r] + 1])
    packed = Vf.verify(np.array(rows), np.array(row0), U, E, W2t, x0, x, ell, u_acc, u_res)
    assert dense["n_acc"].tolist() == packed["n_acc"].tolist()
    assert dense["next_tok"].tolist() == packed["next_tok"].tolist()


def test_residual_falls_back_to_target_when_identical():
    rng = np.random.default_rng(9)
    U, E, W2t, x0, x = _instance(rng, R=1)
    tgt = np.zeros((1, U.shape[1] + 1, U.shape[2]))
    tgt[:, :U.shape[1]] = _draft_logits(U, E, W2t, x0, x)
    res = Vf.residual(tgt, None, U, E, W2t, x0, x, 0, 1, 3)
    pt = np.exp(tgt[0, 1] - np.log(np.exp(tgt[0, 1]).sum()))
    np.testing.assert_allclose(res, pt, rtol=1e-12)


def test_inverse_cdf_boundaries():
    res = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert Vf.inverse_cdf(res, 1e-9) == 1
    assert Vf.inverse_cdf(res, 0.2499) == 1
    assert Vf.inverse_cdf(res, 0.25) == 3          # cumsum must exceed u*Z strictly
    assert Vf.inverse_cdf(res, 0.7501) == 4
    lo, hi = Vf.cdf_interval(res, 3)
    assert (lo, hi) == (0.25, 0.75)
