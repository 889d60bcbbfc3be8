"""Pins for the oracle's RNN head (eq 6): a hand-worked step, gate
saturation at both ends, the zero output projection, an exact reduction to
the (separately pinned) Markov head, and the storage rounding against
torch's bfloat16 conversion."""

import numpy as np
import pytest
import torch

from oracle import rnn as RN
from oracle.sample import markov_sample


def test_hand_worked_two_steps():
    """r = d = 1, W rows (gate, candidate, output) over columns (s, e, h):
    gate 0 -> sigma = 1/2, candidate = e, output = s.  With W1 rows
    e(x0) = 1, e(x1) = 2:  s1 = tanh(1)/2, o1 = tanh(0) = 0;
    s2 = s1/2 + tanh(2)/2, o2 = tanh(s1)."""
    W = np.array([[0.0, 0.0, 0.0], [0.0, 1.0, 0.0], [1.0, 0.0, 0.0]])
    s1, o1 = RN.rnn_step(W, np.zeros((1, 1)), np.array([[1.0]]), np.array([[5.0]]), "f32")
    assert s1[0, 0] == pytest.approx(0.38079707797788244, abs=1e-15)   # tanh(1) / 2
    assert o1[0, 0] == 0.0
    s2, o2 = RN.rnn_step(W, s1, np.array([[2.0]]), np.array([[-3.0]]), "f32")
    assert s2[0, 0] == pytest.approx(0.38079707797788244 / 2 + 0.9640275800758169 / 2, abs=1e-15)
    assert o2[0, 0] == pytest.approx(np.tanh(float(np.float32(0.38079707797788244))), abs=1e-15)


def test_gate_saturation():
    rng = np.random.default_rng(1)
    R, r, d = 3, 4, 5
    W = rng.normal(0, 0.3, size=(3 * r, 2 * r + d))
    s_prev = rng.uniform(-0.9, 0.9, size=(R, r))
    e, h = rng.normal(size=(R, r)), rng.normal(size=(R, d))
    z = np.concatenate([s_prev, e, h], axis=1)
    # a gate of +60 on every row keeps the state; -60 replaces it by the candidate
    Wk = W.copy()
    Wk[:r] = 0.0
    Wk[:r, 2 * r] = 60.0
    h1 = h.copy()
    h1[:, 0] = 1.0
    s, _ = RN.rnn_step(Wk, s_prev, e, h1, "f32")
    np.testing.assert_allclose(s, s_prev, atol=1e-20 + 1e-15)
    h1[:, 0] = -1.0
    s, _ = RN.rnn_step(Wk, s_prev, e, h1, "f32")
    z1 = np.concatenate([s_prev.astype(np.float32).astype(np.float64), e, h1], axis=1)
    np.testing.assert_allclose(s, np.tanh(z1 @ Wk[r:2 * r].T), atol=1e-15)


def _instance(rng, R, gamma, V, r, d, C=16):
    U = rng.normal(0, 2.0, size=(R, gamma, V))
    W2t = rng.normal(0, 1.0 / np.sqrt(r), size=(V, r))
    h = rng.normal(0, 1.0, size=(R, gamma, d))
    x0 = rng.integers(0, V, size=R)
    nC = (V + C - 1) // C
    G = -np.log(-np.log(rng.uniform(size=(R, gamma, nC))))
    g = -np.log(-np.log(rng.uniform(size=(R, gamma, C))))
    return U, W2t, h, x0, G, g


def test_zero_output_projection_means_no_bias():
    rng = np.random.default_rng(2)
    R, gamma, V, r, d = 4, 5, 70, 8, 6
    U, W2t, h, x0, G, g = _instance(rng, R, gamma, V, r, d)
    E = rng.normal(0, 0.5, size=(V, r))
    W = rng.normal(0, 0.3, size=(3 * r, 2 * r + d))
    W[2 * r:] = 0.0
    out = RN.rnn_sample(U, E, W2t, W, h, x0, G, g, "f32")
    ref = markov_sample(U, np.zeros_like(E), W2t, x0, G, g)
    assert out["x"].tolist() == ref["x"].tolist()
    np.testing.assert_allclose(out["lse"], ref["lse"], atol=1e-12)


def test_reduces_to_the_markov_head():
    """W1 entries +-c and an output projection alpha I on the W1 block, alpha =
    atanh(c)/c: tanh(W_o z) = W1[x_{k-1}] exactly, so the RNN head's bias is
    the Markov head's, and the same noise gives the same draws."""
    rng = np.random.default_rng(3)
    R, gamma, V, r, d = 5, 6, 90, 8, 7
    U, W2t, h, x0, G, g = _instance(rng, R, gamma, V, r, d)
    c = 0.5
    E = np.where(rng.random((V, r)) < 0.5, -c, c)
    W = rng.normal(0, 0.3, size=(3 * r, 2 * r + d))
    W[2 * r:] = 0.0
    W[2 * r:, r:2 * r] = np.eye(r) * (np.arctanh(c) / c)
    out = RN.rnn_sample(U, E, W2t, W, h, x0, G, g, "f32")
    ref = markov_sample(U, E, W2t, x0, G, g)
    assert out["x"].tolist() == ref["x"].tolist()
    np.testing.assert_allclose(out["lse"], ref["lse"], atol=1e-9)
    np.testing.assert_allclose(out["o"], E[np.concatenate([x0[:, None], out["x"][:, :-1]], axis=1)], atol=1e-12)


def test_teacher_forcing_follows_the_given_tokens_and_states():
    rng = np.random.default_rng(4)
    R, gamma, V, r, d = 3, 4, 40, 8, 5
    U, W2t, h, x0, G, g = _instance(rng, R, gamma, V, r, d)
    E = rng.normal(0, 0.5, size=(V, r))
    W = rng.normal(0, 0.3, size=(3 * r, 2 * r + d))
    free = RN.rnn_sample(U, E, W2t, W, h, x0, G, g, "bf16")
    forced = RN.rnn_sample(U, E, W2t, W, h, x0, G, g, "bf16", teacher=dict(x=free["x"], s=free["s"]))
    assert forced["x"].tolist() == free["x"].tolist()
    np.testing.assert_allclose(forced["s"], free["s"], atol=1e-15)


def test_bf16_rounding_matches_torch():
    one = 1.0
    cases = np.array([one, one + 2.0 ** -8, one + 3 * 2.0 ** -8, -2.5, 0.0, 1e-30, 65504.0, -3.14159])
    want = np.array([1.0, 1.0, 1.0 + 2.0 ** -6, -2.5, 0.0], dtype=np.float64)
    got = RN.round_storage(cases, "bf16")
    np.testing.assert_array_equal(got[:5], want)          # ties go to the even neighbour
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(0, 3.0, size=4000), rng.uniform(-1, 1, size=4000) * 1e-3])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(RN.round_storage(x, "bf16"), ref)
    np.testing.assert_array_equal(RN.round_storage(cases, "bf16"),
                                  torch.from_numpy(cases.astype(np.float32)).to(torch.bfloat16).double().numpy())


def test_verify_with_bias_vectors_matches_the_markov_rows():
    """The verifier's p_d from explicit bias vectors equals the Markov head's
    when the vectors are the W1 rows of the previous tokens."""
    from oracle import verify as Vf
    rng = np.random.default_rng(8)
    R, gamma, V, r = 4, 5, 60, 8
    U = rng.normal(0, 2.0, size=(R, gamma, V))
    E = rng.normal(0, 0.5, size=(V, r))
    W2t = rng.normal(0, 0.4, size=(V, r))
    x0 = rng.integers(0, V, size=R)
    x = rng.integers(0, V, size=(R, gamma))
    target = rng.normal(0, 2.0, size=(R, gamma + 1, V))
    ell = rng.integers(0, gamma + 1, size=R)
    u_acc, u_res = rng.random((R, gamma)), rng.random(R)
    bvec = E[np.concatenate([x0[:, None], x[:, :-1]], axis=1)]
    a = Vf.verify(target, None, U, E, W2t, x0, x, ell, u_acc, u_res)
    b = Vf.verify(target, None, U, E, W2t, x0, x, ell, u_acc, u_res, bvec=bvec)
    assert a["n_acc"].tolist() == b["n_acc"].tolist() and a["next_tok"].tolist() == b["next_tok"].tolist()
    np.testing.assert_allclose(Vf.analytic_acceptance(target, None, U, E, W2t, x0, x, bvec=bvec),
                               Vf.analytic_acceptance(target, None, U, E, W2t, x0, x), atol=1e-12)
