"""Sequential temperature scaling and calibration metrics, float64 where the
method allows.  Test infrastructure: only tests, the smoke check and the
benchmark's CPU baseline use the oracle.

What is computed (DSpark reading notes, "sequential temperature scaling
(STS)" and the per-position reliability table that follows it;
paper-breakdown page, the confidence-head paragraph):

  * a held-out set of N rollouts, each with the confidence head's logits
    z[n][k] at every drafted position and the accepted prefix length
    n_acc[n] in 0..gamma;
  * the prefix-survival label of position k (1-based) is y_k = [n_acc >= k],
    and the calibrated cumulative product is a_k = a_{k-1} sigmoid(z_k / T_k)
    (a_0 = 1);
  * STS fits T_1, T_2, ... in order: T_k is the grid temperature that
    minimises the ECE of a_k against y_k with T_1..T_{k-1} already fixed;
  * ECE (Guo et al.): M equal-width bins of [0, 1]; the prediction p goes to
    bin min(floor(p M), M - 1); ECE = sum_b |B_b|/N |mean y - mean p| over
    B_b, which is (1/N) sum_b |sum_{n in B_b} (y_n - p_n)|;
  * the per-position ROC-AUC measures how well the raw confidence sigmoid(z_k)
    separates accepted from rejected drafts among the rollouts that reached
    position k (n_acc >= k - 1; accepted iff n_acc >= k), with a tie counted
    as half (the Mann-Whitney statistic); temperature scaling keeps the
    order, so it is the same before and after STS.

Readings where the pages leave a choice:
  * the grid of temperatures and the number of bins are inputs; ties in
    ECE go to the first grid entry;
  * "before STS" is the raw chain, every T = 1;
  * the predictions are evaluated in float32 (as the confidence head
    produces them): sigmoid(x) = 1 / (1 + exp(-x)) on float32 x = z / T, and
    a_k = a_{k-1} * sigmoid(...) rounded to float32; the bin index is taken
    exactly from that float32 value;
  * a position with no rollout reaching it, or with only accepted or only
    rejected drafts, has AUC NaN.
"""

from __future__ import annotations

import numpy as np


def sigmoid32(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)


def ece(p: np.ndarray, y: np.ndarray, n_bins: int) -> float:
    """(1/N) sum_b |sum_{n in b} (y_n - p_n)| with equal-width bins."""
    p = np.asarray(p, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    b = np.minimum(np.floor(p * n_bins), n_bins - 1).astype(np.int64)
    s = np.zeros(n_bins)
    np.add.at(s, b, y - p)
    return float(np.abs(s).sum() / p.shape[0])


def auc_pairs(score: np.ndarray, label: np.ndarray) -> float:
    """P(score of an accepted > score of a rejected) + 1/2 P(equal), by
    comparing every pair (small sets) through sorted counts."""
    score = np.asarray(score, dtype=np.float64)
    label = np.asarray(label, dtype=bool)
    pos, neg = score[label], score[~label]
    if pos.size == 0 or neg.size == 0:
        return float("nan")
    neg_sorted = np.sort(neg)
    below = np.searchsorted(neg_sorted, pos, side="left")
    equal = np.searchsorted(neg_sorted, pos, side="right") - below
    return float((below.sum() + 0.5 * equal.sum()) / (pos.size * neg.size))


def sts_fit(z: np.ndarray, n_acc: np.ndarray, grid: np.ndarray, n_bins: int,
            teacher_T: np.ndarray | None = None) -> dict:
    """T [gamma], ece_before / ece_after [gamma], auc [gamma], and the ECE of
    every grid temperature at every position (ece_grid [gamma][G]).

    teacher_T: when given, position k builds on teacher_T[:k] (another
    implementation's choices) instead of this oracle's own, so that an ECE
    near-tie between two grid entries cannot cascade."""
    z = np.asarray(z, dtype=np.float32)
    N, gamma = z.shape
    n_acc = np.asarray(n_acc)
    grid = np.asarray(grid, dtype=np.float32)
    a = np.ones(N, dtype=np.float32)
    a_raw = np.ones(N, dtype=np.float32)
    T = np.zeros(gamma, dtype=np.float32)
    e_before = np.zeros(gamma)
    e_after = np.zeros(gamma)
    auc = np.zeros(gamma)
    e_grid = np.zeros((gamma, grid.shape[0]))
    for k in range(gamma):
        y = (n_acc >= k + 1).astype(np.float64)
        for t, Tv in enumerate(grid):
            p = (a * sigmoid32(z[:, k] / Tv)).astype(np.float32)
            e_grid[k, t] = ece(p, y, n_bins)
        best = int(np.argmin(e_grid[k]))          # first minimum
        T[k] = grid[best] if teacher_T is None else np.float32(teacher_T[k])
        e_after[k] = e_grid[k, best]
        a_raw = (a_raw * sigmoid32(z[:, k])).astype(np.float32)
        e_before[k] = ece(a_raw, y, n_bins)
        a = (a * sigmoid32(z[:, k] / T[k])).astype(np.float32)
        reach = n_acc >= k
        auc[k] = auc_pairs(z[reach, k], (n_acc >= k + 1)[reach])
    return dict(T=T, ece_before=e_before, ece_after=e_after, auc=auc, ece_grid=e_grid)
