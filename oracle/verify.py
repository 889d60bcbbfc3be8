"""Lossless rejection-sampling verification, float64.

What is computed (DSpark reading notes, the speculative-decoding background
and eq (8a)-(8c), and steps 12-13 of the end-to-end loop; caijizhuo page,
section 四, steps 5-6 of dspark_cycle):

  * target row i of request r predicts draft position i (0-based; the target
    sees the anchor followed by the admitted drafts), and row l_r is the bonus
    row used when every admitted draft is accepted;
  * draft i is accepted with probability min(1, p_t(x_i) / p_d(x_i)), where p_d
    is the drafter's distribution at that position (eq 4 with the Markov bias
    of the previous token) and p_t the target's softmax;
  * the accepted prefix ends at the first rejection, n_r = its length;
  * at the first rejection the next token is drawn from the normalised
    residual max(0, p_t - p_d); when all l_r drafts are accepted it is drawn
    from the bonus row's p_t.  That token is the next round's anchor.

Readings where the pages leave a choice:
  * one uniform per drafted position: accept iff u_acc < ratio, evaluated as
    ln u_acc < ln p_t(x_i) - ln p_d(x_i);
  * the residual / bonus draw is an inverse CDF over the vocabulary in
    ascending order with one uniform: the token is the smallest v with
    cumsum(res)[v] > u_res * Z, Z = sum(res);
  * if Z <= 0 (only when p_t and p_d coincide up to rounding) the draw falls
    back to p_t of the same row;
  * temperature 1 on both sides.

Two more modes (reading notes, the FAQ on greedy,
temperature-0 decoding, and eq (8)-(8c) with the confidence-head paragraph):
  * greedy verification: acceptance becomes an exact-match test of the draft
    token against the target row's argmax; the prefix ends at the first
    mismatch, and the next token is the argmax of the row there (the bonus
    row when every admitted draft matched).  Reading: the argmax takes the
    lowest token index among equal largest logits;
  * the analytic acceptance c*_k = sum_v min(p_d^k(v), p_t^k(v)) of every
    drafted position k (eq 8a; the confidence head's training label),
    target row k against the drafter's distribution at position k.
"""

from __future__ import annotations

import numpy as np

from .common import logsumexp
from .sample import markov_bias


def _target_row(target: np.ndarray, row0, r: int, i: int) -> np.ndarray:
    if row0 is None:
        return target[r, i]
    return target[int(row0[r]) + i]


def draft_logits_at(U: np.ndarray, E: np.ndarray, W2t: np.ndarray, x0: np.ndarray,
                    x: np.ndarray, r: int, i: int, bvec=None) -> np.ndarray:
    """U_i + B_i for request r at draft position i (eq 4's exponent).  With
    bvec [R][gamma][r] (another head's bias vectors, e.g. the RNN head's
    o_i), B_i = bvec[r, i] W2 instead of the Markov head's W1[x_{i-1}] W2."""
    if bvec is not None:
        return U[r, i] + W2t @ np.asarray(bvec[r, i], dtype=np.float64)
    prev = int(x0[r]) if i == 0 else int(x[r, i - 1])
    return U[r, i] + markov_bias(E, W2t, np.array([prev]))[0]


def accept_log_ratios(target, row0, U, E, W2t, x0, x, ell, bvec=None):
    """For each request, ln p_t(x_i) - ln p_d(x_i) for i < l_r (a list of arrays)."""
    R = U.shape[0]
    out = []
    for r in range(R):
        vals = []
        for i in range(int(ell[r])):
            lt = _target_row(target, row0, r, i)
            ld = draft_logits_at(U, E, W2t, x0, x, r, i, bvec)
            xi = int(x[r, i])
            vals.append((lt[xi] - logsumexp(lt)) - (ld[xi] - logsumexp(ld)))
        out.append(np.array(vals))
    return out


def first_rejection(log_ratio: np.ndarray, u: np.ndarray) -> int:
    """Length of the accepted prefix: the index of the first i with
    ln u_i >= ln ratio_i, or the number of positions if none."""
    for i in range(log_ratio.shape[0]):
        if not (np.log(float(u[i])) < log_ratio[i]):
            return i
    return int(log_ratio.shape[0])


def residual(target, row0, U, E, W2t, x0, x, r: int, n: int, ell_r: int, bvec=None) -> np.ndarray:
    """The distribution (unnormalised) the next token is drawn from."""
    lt = _target_row(target, row0, r, n)
    pt = np.exp(lt - logsumexp(lt))
    if n >= ell_r:
        return pt                                   # bonus row: p_t itself
    ld = draft_logits_at(U, E, W2t, x0, x, r, n, bvec)
    pd = np.exp(ld - logsumexp(ld))
    res = np.maximum(0.0, pt - pd)
    if not (res.sum() > 0.0):
        return pt                                   # p_t == p_d up to rounding
    return res


def inverse_cdf(res: np.ndarray, u: float) -> int:
    """Smallest v with cumsum(res)[v] > u * sum(res)."""
    cdf = np.cumsum(res)
    t = float(u) * cdf[-1]
    v = int(np.searchsorted(cdf, t, side="right"))
    return min(v, res.shape[0] - 1)


def verify(target, row0, U, E, W2t, x0, x, ell, u_acc, u_res, n_teacher=None, bvec=None) -> dict:
    """Accepted lengths n_acc [R] and next tokens next_tok [R].

    n_teacher: when given, the residual draw uses these accepted lengths instead
    of the oracle's own (to check another implementation past a near-tie)."""
    R = U.shape[0]
    logr = accept_log_ratios(target, row0, U, E, W2t, x0, x, ell, bvec)
    n_acc = np.zeros(R, dtype=np.int64)
    next_tok = np.zeros(R, dtype=np.int64)
    margins = []
    for r in range(R):
        n = first_rejection(logr[r], u_acc[r])
        n_acc[r] = n
        if logr[r].shape[0]:
            margins.append(np.abs(np.log(u_acc[r, :logr[r].shape[0]].astype(np.float64)) - logr[r]))
        n_use = n if n_teacher is None else int(n_teacher[r])
        res = residual(target, row0, U, E, W2t, x0, x, r, n_use, int(ell[r]), bvec)
        next_tok[r] = inverse_cdf(res, u_res[r])
    return dict(n_acc=n_acc, next_tok=next_tok, log_ratio=logr, margins=margins)


def cdf_interval(res: np.ndarray, v: int):
    """[cdf(v-1), cdf(v)) as fractions of the total: the u-range that draws v."""
    cdf = np.cumsum(res)
    Z = cdf[-1]
    lo = cdf[v - 1] / Z if v > 0 else 0.0
    return lo, cdf[v] / Z


def row_argmax(logits: np.ndarray) -> int:
    """Lowest index among the largest entries."""
    return int(np.argmax(logits))     # numpy returns the first maximum


def verify_greedy(target, row0, x, ell) -> dict:
    """Temperature-0 verification: n_r = the first i < l_r with
    x_i != argmax(target row i) (l_r if none), next = argmax(target row n_r)."""
    x = np.asarray(x)
    R = x.shape[0]
    n_acc = np.zeros(R, dtype=np.int64)
    next_tok = np.zeros(R, dtype=np.int64)
    for r in range(R):
        L = int(ell[r])
        n = L
        for i in range(L):
            if int(x[r, i]) != row_argmax(_target_row(target, row0, r, i)):
                n = i
                break
        n_acc[r] = n
        next_tok[r] = row_argmax(_target_row(target, row0, r, n))
    return dict(n_acc=n_acc, next_tok=next_tok)


def analytic_acceptance(target, row0, U, E, W2t, x0, x, lse=None, bvec=None) -> np.ndarray:
    """c*[r, k] = sum_v min(p_d(v), p_t(v)) at every drafted position k, in
    float64.  p_d is the drafter's softmax at position k (U_k plus the Markov
    bias of x_{k-1}); its log-normaliser is computed here, or taken from
    `lse` [R][gamma] when given (to check another implementation that is
    handed the sampler's normalisers).  p_t is the softmax of target row k."""
    R, gamma = np.asarray(x).shape
    out = np.zeros((R, gamma), dtype=np.float64)
    for r in range(R):
        for k in range(gamma):
            lt = np.asarray(_target_row(target, row0, r, k), dtype=np.float64)
            pt = np.exp(lt - logsumexp(lt))
            ld = draft_logits_at(U, E, W2t, x0, x, r, k, bvec).astype(np.float64)
            nd = logsumexp(ld) if lse is None else float(lse[r, k])
            pd = np.exp(ld - nd)
            out[r, k] = float(np.minimum(pd, pt).sum())
    return out
