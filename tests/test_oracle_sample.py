"""Pins for the oracle's Markov-head sampler and confidence head: textbook
reductions, closed forms and the sampled distribution (chi-square)."""

import numpy as np
import pytest
from scipy import stats

from oracle import common, confidence as Cf
from oracle.sample import markov_bias, markov_sample, sample_position, token_gaps


def gumbels(rng, shape):
    return -np.log(-np.log(rng.uniform(size=shape)))


def test_logsumexp_closed_form():
    l = np.full((2, 100), 3.0)
    np.testing.assert_allclose(common.logsumexp(l, axis=1), 3.0 + np.log(100.0), rtol=1e-15)
    l = np.array([[0.0, -np.inf, np.log(3.0)]])
    assert common.logsumexp(l, axis=1)[0] == pytest.approx(np.log(4.0), rel=1e-15)


def test_bf16_upcast_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], dtype=np.uint16)
    got = common.as_f64(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -1.0
    assert got[2] == pytest.approx(3.140625, rel=0)
    assert got[3] == 2.0 ** -133
    assert got[4] == pytest.approx(3.3895313892515355e38, rel=1e-15)


def test_bias_one_hot_rows_select_columns_of_w2():
    """eq 5: B(prev, .) = W1[prev] W2.  With W1 rows one-hot (row p = e_{p mod r})
    the bias is the (p mod r)-th row of W2, i.e. column (p mod r) of W2t."""
    rng = np.random.default_rng(0)
    V, r = 50, 8
    E = np.zeros((V, r))
    E[np.arange(V), np.arange(V) % r] = 1.0
    W2t = rng.normal(size=(V, r))
    prev = np.array([3, 12, -1, 49])
    B = markov_bias(E, W2t, prev)
    np.testing.assert_array_equal(B[0], W2t[:, 3])
    np.testing.assert_array_equal(B[1], W2t[:, 12 % r])
    np.testing.assert_array_equal(B[2], 0.0)
    np.testing.assert_array_equal(B[3], W2t[:, 49 % r])


@pytest.mark.parametrize("C,V", [(64, 50), (16, 12), (16, 16)])
def test_single_chunk_reduces_to_textbook_gumbel_max(C, V):
    rng = np.random.default_rng(1)
    R, r = 64, 4
    U = rng.normal(0, 2, size=(R, 1, V))
    E = rng.normal(0, 0.5, size=(V, r))
    W2t = rng.normal(0, 0.5, size=(V, r))
    x0 = rng.integers(-1, V, size=R)
    G = gumbels(rng, (R, 1, 1))
    g = gumbels(rng, (R, 1, C))
    out = markov_sample(U, E, W2t, x0, G, g)
    for i in range(R):
        bias = np.zeros(V) if x0[i] < 0 else sum(E[x0[i], k] * W2t[:, k] for k in range(r))
        l = U[i, 0] + bias
        assert out["x"][i, 0] == int(np.argmax(l + g[i, 0, :V]))
        m = l.max()
        assert out["lse"][i, 0] == pytest.approx(m + np.log(np.exp(l - m).sum()), rel=1e-13)
        assert out["logit"][i, 0] == pytest.approx(l[out["x"][i, 0]], rel=1e-13, abs=1e-13)


@pytest.mark.parametrize("C,V,sizes", [(64, 150, [64.0, 64.0, 22.0]),
                                       (16, 40, [16.0, 16.0, 8.0])])
def test_chunk_log_normalisers_closed_form(C, V, sizes):
    R = 1          # two full chunks and a short tail
    U = np.full((R, 1, V), 0.7)
    E = np.zeros((V, 4))
    W2t = np.zeros((V, 4))
    st = sample_position(U[:, 0], E, W2t, np.array([-1]), np.zeros((1, 3)), np.zeros((1, C)))
    np.testing.assert_allclose(st["chunk_score"][0], 0.7 + np.log(sizes), rtol=1e-14)
    assert st["lse"][0] == pytest.approx(0.7 + np.log(float(V)), rel=1e-14)
    # equal chunk scores: the lowest chunk wins; equal in-chunk scores: lowest offset
    st = sample_position(U[:, 0], E, W2t, np.array([-1]), -np.log([sizes]), np.zeros((1, C)))
    assert st["token"][0] == 0
    # a dominant chunk Gumbel picks that chunk; the in-chunk Gumbels pick the offset
    gg = np.zeros((1, C))
    gg[0, 5] = 1.0
    st = sample_position(U[:, 0], E, W2t, np.array([-1]), np.array([[0.0, 50.0, 0.0]]), gg)
    assert st["token"][0] == C + 5


@pytest.mark.parametrize("with_bias,C", [(False, 64), (True, 64), (True, 16)])
def test_two_level_draw_follows_softmax(with_bias, C):
    """The sampled token follows p(v) = softmax(U + B)(v) (chi-square), over a
    vocabulary of 200 = 3 full chunks of 64 and a ragged tail of 8 (or 12
    full chunks of 16 and a tail of 8)."""
    rng = np.random.default_rng(42 + with_bias + C)
    V, r, R = 200, 6, 60000
    base = rng.normal(0, 1.0, size=V)
    base[17] += 3.0
    base[130] += 2.5
    E = rng.normal(0, 0.5, size=(V, r)) if with_bias else np.zeros((V, r))
    W2t = rng.normal(0, 0.5, size=(V, r)) if with_bias else np.zeros((V, r))
    prev = 33
    l = base + (E[prev] @ W2t.T)
    p = np.exp(l - l.max())
    p /= p.sum()
    U = np.broadcast_to(base, (R, 1, V)).copy()
    x0 = np.full(R, prev)
    G = gumbels(rng, (R, 1, (V + C - 1) // C))
    g = gumbels(rng, (R, 1, C))
    x = markov_sample(U, E, W2t, x0, G, g)["x"][:, 0]
    counts = np.bincount(x, minlength=V).astype(float)
    exp = R * p
    big = exp >= 5.0
    obs, ex = counts[big], exp[big]
    if np.any(~big):
        obs, ex = np.append(obs, counts[~big].sum()), np.append(ex, exp[~big].sum())
    assert stats.chisquare(obs, ex).pvalue > 1e-3


def test_zero_bias_head_samples_positions_independently():
    """W2 = 0 (no Markov head): position k depends on U_k and its own noise only."""
    rng = np.random.default_rng(3)
    R, gamma, V, r = 5, 4, 130, 8
    U = rng.normal(0, 2, size=(R, gamma, V))
    E = rng.normal(size=(V, r))
    W2t = np.zeros((V, r))
    G = gumbels(rng, (R, gamma, 3))
    g = gumbels(rng, (R, gamma, 64))
    a = markov_sample(U, E, W2t, rng.integers(0, V, R), G, g)
    b = markov_sample(U, E, W2t, rng.integers(0, V, R), G, g)
    np.testing.assert_array_equal(a["x"], b["x"])


def test_teacher_forcing_uses_the_given_previous_tokens():
    rng = np.random.default_rng(4)
    R, gamma, V, r = 3, 3, 70, 4
    U = rng.normal(0, 2, size=(R, gamma, V))
    E = rng.normal(size=(V, r))
    W2t = rng.normal(size=(V, r))
    x0 = rng.integers(0, V, R)
    G = gumbels(rng, (R, gamma, 2))
    g = gumbels(rng, (R, gamma, 64))
    teacher = rng.integers(0, V, (R, gamma))
    out = markov_sample(U, E, W2t, x0, G, g, teacher_x=teacher, keep_steps=True)
    st = sample_position(U[:, 2], E, W2t, teacher[:, 1], G[:, 2], g[:, 2])
    np.testing.assert_array_equal(out["x"][:, 2], st["token"])
    cg, ig = token_gaps(out["steps"][2], g[:, 2], out["x"][:, 2])
    assert np.all(cg == 0) and np.all(ig == 0)
    other = (out["x"][:, 2] + 1) % V
    cg, ig = token_gaps(out["steps"][2], g[:, 2], other)
    assert np.all((cg > 0) | (ig > 0))


# ----------------------------------------------------------------- confidence

def test_confidence_zero_weights_is_one_half():
    R, gamma, d, r, V = 2, 3, 5, 4, 10
    out = Cf.confidence(np.ones((R, gamma, d)), np.zeros(d + r), np.ones((V, r)),
                        np.array([1, 2]), np.zeros((R, gamma), dtype=np.int64))
    np.testing.assert_array_equal(out["c"], 0.5)


def test_confidence_closed_form_and_previous_token_index():
    """eq 7 with one-hot inputs: z = w_h[i] * a + w_e[prev mod r], where prev is
    the anchor at position 1 and the previous draft afterwards."""
    R, gamma, d, r, V = 1, 3, 6, 4, 20
    h = np.zeros((R, gamma, d))
    h[0, :, 2] = [1.0, 2.0, -1.0]
    w = np.zeros(d + r)
    w[2] = 0.5
    w[d:] = [10.0, 20.0, 30.0, 40.0]
    E = np.zeros((V, r))
    E[np.arange(V), np.arange(V) % r] = 1.0
    x0 = np.array([5])                 # 5 mod 4 = 1 -> 20
    x = np.array([[6, 7, 8]])          # prev for k=2: 6 -> 30; k=3: 7 -> 40
    out = Cf.confidence(h, w, E, x0, x)
    np.testing.assert_allclose(out["z"][0], [0.5 + 20.0, 1.0 + 30.0, -0.5 + 40.0])
    out = Cf.confidence(h, w, E, np.array([-1]), x)
    assert out["z"][0, 0] == 0.5


def test_confidence_temperature():
    R, gamma, d, r, V = 1, 2, 1, 1, 4
    h = np.full((R, gamma, d), 2.0)
    w = np.array([1.0, 0.0])
    out = Cf.confidence(h, w, np.zeros((V, r)), np.array([0]), np.zeros((1, 2), dtype=np.int64),
                        T=np.array([1.0, 2.0], dtype=np.float32))
    assert out["c"][0, 0] == pytest.approx(1.0 / (1.0 + np.exp(-2.0)), rel=1e-15)
    assert out["c"][0, 1] == pytest.approx(1.0 / (1.0 + np.exp(-1.0)), rel=1e-15)


def test_sigmoid_extremes_and_symmetry():
    t = np.array([-800.0, -20.0, 0.0, 20.0, 800.0])
    s = Cf.sigmoid(t)
    assert np.all(np.isfinite(s))
    assert s[0] == 0.0 or s[0] > 0.0
    assert s[-1] == 1.0 and s[2] == 0.5
    np.testing.assert_allclose(s + Cf.sigmoid(-t), 1.0, rtol=1e-15)
