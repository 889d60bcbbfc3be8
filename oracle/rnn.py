"""RNN-head draft sampling over a gamma-block, float64.  Test infrastructure:
only tests, the smoke check and the benchmark's CPU baseline use the oracle.

What is computed (DSpark reading notes, "implementation two: the RNN head",
eq (6); atlas chapter, the two heads):

  * the head keeps a state s_k in R^r over the block, s_0 = 0;
  * at position k it concatenates z_k = [s_{k-1}; W1[x_{k-1}]; h_k] (length
    2r + d) and applies one packed projection W = [W_g; W_c; W_o]
    ([3r][2r + d]), split into gate, candidate and output parts;
  * s_k = sigma(W_g z_k) * s_{k-1} + (1 - sigma(W_g z_k)) * tanh(W_c z_k);
  * the bias is B_k = tanh(W_o z_k) W2: the r-vector o_k = tanh(W_o z_k)
    takes the place of W1[x_{k-1}] in eq (5)'s product, and x_k is drawn
    from softmax(U_k + B_k) as with the Markov head (the same exact
    two-level Gumbel-max, oracle.sample).

Readings where the pages leave a choice:
  * the first position's previous token is the anchor x0; x0 = -1 gives a
    W1 part of zeros (as the Markov head's bias 0);
  * operand precision: with bf16 storage, z enters the projection in bf16 --
    its W1 and h parts are stored that way, and the state (carried in
    float32 between positions) is rounded to bf16 (to nearest, ties to even)
    where it enters z; o_k is rounded the same way before the bias product.
    With fp32 storage nothing is rounded beyond float32.  The head's
    arithmetic is otherwise exact (float64 here).
"""

from __future__ import annotations

import numpy as np

from .sample import sample_with_bias


def round_storage(x: np.ndarray, store: str) -> np.ndarray:
    """x rounded to float32, then (bf16 storage) to bfloat16 by
    round-to-nearest-even on the float32 bit pattern; returned as float64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if store == "f32":
        return f.astype(np.float64)
    assert store == "bf16"
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isfinite(f), out, f.astype(np.float64))


def sigmoid(y: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * y))


def rnn_step(W: np.ndarray, s_prev: np.ndarray, e_prev: np.ndarray, h_k: np.ndarray, store: str):
    """One step of eq (6) for every request: returns (s_k, o_k) in float64.
    W [3r][2r+d]; s_prev, e_prev [R][r]; h_k [R][d]."""
    r = s_prev.shape[1]
    z = np.concatenate([round_storage(s_prev, store), e_prev, h_k], axis=1)   # [R][2r+d]
    y = z @ W.T                                                               # [R][3r]
    gate = sigmoid(y[:, :r])
    s = gate * s_prev + (1.0 - gate) * np.tanh(y[:, r:2 * r])
    o = np.tanh(y[:, 2 * r:])
    return s, o


def rnn_sample(U, E, W2t, W, h, x0, G, g, store: str, teacher: dict | None = None) -> dict:
    """The gamma-step loop with the RNN head.  U [R][gamma][V], E = W1 [V][r],
    W2t [V][r], W [3r][2r+d], h [R][gamma][d] (float64 values of the stored
    arrays); G [R][gamma][nC], g [R][gamma][C].

    teacher: {"x": [R][gamma], "s": [R][gamma][r]} from another implementation;
    position k then takes its previous token and previous state from there,
    so that a near-tie cannot cascade.  With "o" [R][gamma][r] as well, the
    draw at position k uses that bias vector (already in storage precision)
    instead of this oracle's own rounded o_k, so that a case on a rounding
    boundary is checked in the head and not again in the draw."""
    R, gamma, V = U.shape
    r = E.shape[1]
    x = np.zeros((R, gamma), dtype=np.int64)
    lse = np.zeros((R, gamma))
    logit = np.zeros((R, gamma))
    S = np.zeros((R, gamma, r))
    O = np.zeros((R, gamma, r))
    steps = []
    prev = np.asarray(x0, dtype=np.int64)
    s_prev = np.zeros((R, r))
    for k in range(gamma):
        e_prev = np.zeros((R, r))
        live = prev >= 0
        e_prev[live] = E[prev[live]]
        s, o = rnn_step(W, s_prev, e_prev, h[:, k, :], store)
        S[:, k] = s
        O[:, k] = o
        o_used = (np.asarray(teacher["o"][:, k], dtype=np.float64) if teacher is not None and "o" in teacher
                  else round_storage(o, store))
        B = o_used @ W2t.T
        st = sample_with_bias(U[:, k, :], B, G[:, k, :], g[:, k, :])
        x[:, k] = st["token"]
        lse[:, k] = st["lse"]
        logit[:, k] = st["logit"]
        steps.append(st)
        if teacher is None:
            prev, s_prev = st["token"], s
        else:
            prev = np.asarray(teacher["x"][:, k], dtype=np.int64)
            s_prev = np.asarray(teacher["s"][:, k], dtype=np.float64)
    return dict(x=x, lse=lse, logit=logit, s=S, o=O, steps=steps)
