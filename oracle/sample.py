"""Markov-head draft sampling over a gamma-block, float64.

What is computed (DSpark reading notes, eq (4) and eq (5); caijizhuo page,
section 二 and the sequential loop of dspark_cycle in section 四):

  * position k draws x_k from p_k(v) proportional to exp(U_k(v) + B_k(v));
  * the Markov head's bias depends on the previous token only and is low rank:
    B(x_{k-1}, .) = W1[x_{k-1}] W2, a row lookup in W1 (V x r) times W2 (r x V);
  * position 1 conditions on the anchor x0 (the notes' eq (4) conditions on
    x0 and the symbol table calls x0 the previous round's bonus token); an
    anchor of -1 selects the caijizhuo page's variant, where the first step
    uses the raw scores (bias 0);
  * only the sampled token is carried from one position to the next.

The pages only say "sample"; the draw is made here as an exact two-level
Gumbel-max.  The vocabulary is cut into chunks of C consecutive tokens (the
last one may be short).  With LSE_c the log-sum-exp of the logits in chunk c,
the chunk is argmax_c (LSE_c + G_c), and the token is the in-chunk argmax of
l_v + g_i, i the token's offset inside its chunk.  The maximum of
Gumbel-perturbed logits over a set is itself Gumbel with location the set's
log-sum-exp, so the chunk is drawn with probability exp(LSE_c)/Z and the
token inside it with probability exp(l_v)/exp(LSE_c): the product is p_k(v).
The in-chunk Gumbels g are drawn once per position and reused by every chunk;
only the winning chunk's in-chunk draw is ever used, so this is still exact.
With a single chunk (V <= C) the draw is the textbook argmax(l + g).
Ties go to the lowest chunk, then the lowest offset.

W2 is passed as W2t with shape [V][r] (row v of W2t is column v of W2).

Parity: pinned in distribution (chi-square against softmax), by the
single-chunk reduction to textbook Gumbel-max and by closed forms for the bias
(one-hot W1 rows select rows of W2t) and the normaliser.  The pages' own
Markov example prints output probabilities but no logits, so agreement with
that example is parity unpinned.
"""

from __future__ import annotations

import numpy as np

from .common import logsumexp


def markov_bias(E: np.ndarray, W2t: np.ndarray, prev: np.ndarray) -> np.ndarray:
    """B[r, :] = W1[prev_r] W2 (eq 5); a row of zeros where prev_r = -1."""
    R = prev.shape[0]
    V = W2t.shape[0]
    B = np.zeros((R, V), dtype=np.float64)
    live = prev >= 0
    if np.any(live):
        B[live] = E[prev[live]] @ W2t.T   # (n x r) @ (r x V)
    return B


def sample_position(U_k: np.ndarray, E: np.ndarray, W2t: np.ndarray, prev: np.ndarray,
                    G_k: np.ndarray, g_k: np.ndarray) -> dict:
    """One position for every request.  U_k [R][V], G_k [R][nC], g_k [R][C]."""
    return sample_with_bias(U_k, markov_bias(E, W2t, prev), G_k, g_k)


def sample_with_bias(U_k: np.ndarray, B_k: np.ndarray, G_k: np.ndarray, g_k: np.ndarray) -> dict:
    """One position for every request, given its bias B_k [R][V] (eq 4 with
    any head's B_k)."""
    R, V = U_k.shape
    C = g_k.shape[1]
    nC = G_k.shape[1]
    assert nC == (V + C - 1) // C
    l = U_k + B_k                                # exponent of eq (4)
    lse = logsumexp(l, axis=1)                   # log of eq (4)'s denominator
    lpad = np.full((R, nC * C), -np.inf)
    lpad[:, :V] = l
    lpad = lpad.reshape(R, nC, C)
    chunk_lse = logsumexp(lpad, axis=2)          # [R][nC]
    chunk_score = chunk_lse + G_k
    c_star = np.argmax(chunk_score, axis=1)      # first maximum = lowest chunk
    inner = lpad[np.arange(R), c_star, :] + g_k  # [R][C]; padded slots stay -inf
    t_star = np.argmax(inner, axis=1)
    token = c_star * C + t_star
    return dict(l=l, lse=lse, chunk_score=chunk_score, token=token.astype(np.int64),
                logit=l[np.arange(R), token], lpad=lpad)


def token_gaps(step: dict, g_k: np.ndarray, token: np.ndarray):
    """How far a proposed token is from the oracle's draw, in perturbed score.

    Returns (chunk_gap, inner_gap): the chunk-level score of the oracle's chunk
    minus that of the token's chunk, and the best in-chunk perturbed score of
    the token's chunk minus the token's own.  Both are 0 when the token is the
    oracle's draw."""
    C = g_k.shape[1]
    R = token.shape[0]
    rows = np.arange(R)
    c = token // C
    t = token % C
    S = step["chunk_score"]
    chunk_gap = S.max(axis=1) - S[rows, c]
    inner = step["lpad"][rows, c, :] + g_k
    inner_gap = inner.max(axis=1) - inner[rows, t]
    return chunk_gap, inner_gap


def markov_sample(U: np.ndarray, E: np.ndarray, W2t: np.ndarray, x0: np.ndarray,
                  G: np.ndarray, g: np.ndarray, teacher_x: np.ndarray | None = None,
                  keep_steps: bool = False) -> dict:
    """The gamma-step sequential loop.  U [R][gamma][V] float64.

    teacher_x: when given, position k conditions on teacher_x[:, k-1] instead
    of the oracle's own previous draw (used to check another implementation
    position by position without letting one near-tie cascade)."""
    R, gamma, V = U.shape
    x = np.zeros((R, gamma), dtype=np.int64)
    lse = np.zeros((R, gamma))
    logit = np.zeros((R, gamma))
    steps = []
    prev = np.asarray(x0, dtype=np.int64)
    for k in range(gamma):
        st = sample_position(U[:, k, :], E, W2t, prev, G[:, k, :], g[:, k, :])
        x[:, k] = st["token"]
        lse[:, k] = st["lse"]
        logit[:, k] = st["logit"]
        if keep_steps:
            steps.append(st)
        prev = (np.asarray(teacher_x[:, k], dtype=np.int64) if teacher_x is not None
                else st["token"])
    out = dict(x=x, lse=lse, logit=logit)
    if keep_steps:
        out["steps"] = steps
    return out
