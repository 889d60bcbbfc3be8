"""Pins of the oracle's whole-round composition, oracle/round.py run_round.

run_round chains the pinned stages in the order of the end-to-end decode
loop (reading notes, "full decode loop" pseudocode, steps 3-13; caijizhuo
page, dspark_cycle steps 3-6).  Two kinds of pin:

  * a special case whose every output follows from the definitions by hand:
    with W1 = 0 the Markov bias vanishes, so each position is an independent
    two-level Gumbel-max draw from softmax(U_k) (recomputed here with plain
    Python loops over the stored layout of G, so a transposed G fails), the
    confidence reduces to sigmoid(w_h . h_k / T_k), and a target whose rows
    0..gamma-1 equal the drafter's logits makes every accept ratio exactly 1,
    so every admitted draft is accepted (n = ell) and the next token is the
    inverse-CDF draw from the bonus row ell_r (not row gamma);
  * the general case against the stage-by-stage composition, with the chunk
    Gumbels gathered request-major by explicit indexing.
"""

import math

import numpy as np
import pytest

from oracle.common import as_f64
from oracle.confidence import confidence
from oracle.round import run_round
from oracle.sample import markov_sample
from oracle.schedule import admit
from oracle.verify import verify
from semi_ar_draft_round_amd import workloads as W

CASES = [
    W.BY_NAME["tiny_r1_g4_v1024_f32"],
    W.custom("round_pin_r3_g3_v203_bf16", R=3, gamma=3, V=203, r=32, d=64, seed=71, temperatures=True),
    W.custom("round_pin_r4_g5_v100_f32", R=4, gamma=5, V=100, r=8, d=16, dtype="f32", seed=72),
]


def _gumbel_max_by_hand(l, G_of_chunk, g):
    """Two-level Gumbel-max over one row of logits l (Python floats): chunks
    of 16, chunk = argmax(LSE_c + G_c), token = in-chunk argmax(l_v + g[v % 16]);
    first maximum wins at both levels."""
    V = len(l)
    nC = (V + 15) // 16
    best_c, best_s = -1, -math.inf
    for c in range(nC):
        vals = l[16 * c: min(V, 16 * c + 16)]
        m = max(vals)
        lse = m + math.log(sum(math.exp(v - m) for v in vals))
        s = lse + G_of_chunk(c)
        if s > best_s:
            best_c, best_s = c, s
    lo = 16 * best_c
    best_t, best_v = -1, -math.inf
    for t in range(min(16, V - lo)):
        s = l[lo + t] + g[t]
        if s > best_v:
            best_t, best_v = t, s
    return lo + best_t


def _inverse_cdf_by_hand(logits, u):
    m = max(logits)
    p = [math.exp(v - m) for v in logits]
    Z = math.fsum(p)
    acc = 0.0
    for v, pv in enumerate(p):
        acc += pv
        if acc > u * Z:
            return v
    return len(p) - 1


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_round_special_case_no_bias_self_target(w):
    inp = W.make_inputs(w)
    dt = w.dtype
    inp.E[:] = 0                                    # W1 = 0: B_k = 0 and no W1 part in z
    # target rows 0..gamma-1 = the drafter's logits (the same stored bits); the
    # bonus row gamma keeps its own values
    inp.target[:, :w.gamma, :] = inp.U
    out = run_round(inp)
    U = as_f64(inp.U, dt)
    h = as_f64(inp.h, dt)
    wc = as_f64(inp.w_conf, dt)
    tgt = as_f64(inp.target, dt)
    R, gamma, V, d = w.R, w.gamma, w.V, w.d
    for i in range(R):
        for k in range(gamma):
            want = _gumbel_max_by_hand(list(U[i, k]), lambda c: float(inp.G[k, c, i]), list(inp.g[i, k]))
            assert out["x"][i, k] == want, (i, k)
            z = math.fsum(float(wc[j]) * float(h[i, k, j]) for j in range(d))
            T = 1.0 if inp.T is None else float(inp.T[k])
            assert out["z"][i, k] == pytest.approx(z, rel=1e-12, abs=1e-12)
            assert out["c"][i, k] == pytest.approx(1.0 / (1.0 + math.exp(-z / T)), rel=1e-12)
    # the scheduler sees the confidences as fp32, exactly as the GPU hands them over
    ref = admit(np.asarray(out["c"], dtype=np.float32), inp.sps)
    assert out["ell"].tolist() == ref["ell"].tolist()
    assert out["A"] == ref["A"] and out["theta_best"] == ref["theta_best"]
    # ratio p_t / p_d = 1 everywhere: accept iff u < 1, always true for u in (0, 1)
    assert out["n_acc"].tolist() == out["ell"].tolist()
    for i in range(R):
        L = int(out["ell"][i])
        assert out["next_tok"][i] == _inverse_cdf_by_hand(list(tgt[i, L]), float(inp.u_res[i])), i


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_round_equals_stagewise_composition(w):
    inp = W.make_inputs(w)
    dt = w.dtype
    out = run_round(inp)
    R, gamma, nC = w.R, w.gamma, w.n_chunks
    Greq = np.empty((R, gamma, nC), dtype=np.float32)
    for i in range(R):
        for k in range(gamma):
            for c in range(nC):
                Greq[i, k, c] = inp.G[k, c, i]
    U = as_f64(inp.U, dt)
    E = as_f64(inp.E, dt)
    W2t = as_f64(inp.W2t, dt)
    x0 = inp.x0.astype(np.int64)
    s = markov_sample(U, E, W2t, x0, Greq, inp.g)
    cf = confidence(as_f64(inp.h, dt), as_f64(inp.w_conf, dt), E, x0, s["x"], inp.T)
    sc = admit(cf["c"].astype(np.float32), inp.sps)
    vf = verify(as_f64(inp.target, dt), None, U, E, W2t, x0, s["x"], sc["ell"], inp.u_acc, inp.u_res)
    np.testing.assert_array_equal(out["x"], s["x"])
    np.testing.assert_array_equal(out["lse"], s["lse"])
    np.testing.assert_array_equal(out["c"], cf["c"])
    np.testing.assert_array_equal(out["ell"], sc["ell"])
    assert out["A"] == sc["A"]
    np.testing.assert_array_equal(out["n_acc"], vf["n_acc"])
    np.testing.assert_array_equal(out["next_tok"], vf["next_tok"])


def test_round_on_a_request_subset_is_the_subset_of_the_round():
    """The bounded CPU baseline times run_round on a request subset: the
    per-request stages of a subset equal those rows of the whole round."""
    w = CASES[1]
    inp = W.make_inputs(w)
    whole = run_round(inp)
    part = run_round(inp, requests=[0, 2])
    np.testing.assert_array_equal(part["x"], whole["x"][[0, 2]])
    np.testing.assert_array_equal(part["c"], whole["c"][[0, 2]])
