"""Confidence head with per-position temperature, float64.

What is computed (DSpark reading notes, eq (7) and the sequential temperature
scaling paragraph; the LLM-infra atlas chapter, section 4.2):

  c_k = sigma(w^T [h_k ; W1[x_{k-1}]])

one linear projection of the backbone hidden state h_k concatenated with the
Markov embedding of the previous draft token, then a sigmoid.  The weight
vector is ordered as the concatenation is: the first d entries multiply h_k,
the last r entries multiply W1[x_{k-1}].

Readings where the pages leave a choice:
  * the token fed to the head is x_{k-1} (eq 7, and the atlas chapter), not the
    token just sampled at k as the caijizhuo pseudocode's keyword suggests;
    this keeps c_k independent of x_k, which the non-anticipation argument of
    Appendix A needs.  Position 1 uses the anchor x0; an anchor of -1 makes the
    W1 part zero.
  * sequential temperature scaling divides the logit by T_k before the
    sigmoid: c~_k = sigma(z_k / T_k), an order-preserving rescaling; T = None
    means T_k = 1.
"""

from __future__ import annotations

import numpy as np


def sigmoid(t: np.ndarray) -> np.ndarray:
    """1/(1+e^-t), evaluated without overflow on either side."""
    t = np.asarray(t, dtype=np.float64)
    out = np.empty_like(t)
    pos = t >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-t[pos]))
    e = np.exp(t[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def confidence(h: np.ndarray, w: np.ndarray, E: np.ndarray, x0: np.ndarray,
               x: np.ndarray, T: np.ndarray | None = None) -> dict:
    """h [R][gamma][d], w [d+r], E [V][r], x0 [R], x [R][gamma] (drafted tokens).

    Returns z [R][gamma] (the pre-sigmoid logit, before temperature) and c."""
    R, gamma, d = h.shape
    r = E.shape[1]
    assert w.shape[0] == d + r
    prev = np.concatenate([np.asarray(x0, dtype=np.int64)[:, None],
                           np.asarray(x, dtype=np.int64)[:, :gamma - 1]], axis=1)
    emb = np.zeros((R, gamma, r))
    live = prev >= 0
    emb[live] = E[prev[live]]
    z = h @ w[:d] + emb @ w[d:]
    Tk = np.ones(gamma) if T is None else np.asarray(T, dtype=np.float64)
    c = sigmoid(z / Tk[None, :])
    return dict(z=z, c=c)
