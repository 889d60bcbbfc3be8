"""Hardware-aware prefix scheduler (Algorithm 1), exact arithmetic.

What is computed (DSpark reading notes, "hardware-aware prefix scheduler":
the objective Theta = tau * SPS(B), Algorithm 1 steps 1-6, Lemmas 1-2 and
step 3 of the optimality sketch, Appendix A's eq (9)-(10); caijizhuo page,
sections 三 and 四 (the single-request admit); atlas chapter, section 4.3):

  1. a_{r,j} = prod_{i<=j} c_{r,i}                  (cumulative survival)
  2. pool every (r, j) with a_{r,j} > 0, sort by a_{r,j}, largest first
  3-4. start from B = R (one anchor slot per request), tau = R,
       Theta_best = R * SPS(R), every l_r = 0
  5. walk the sorted pool: admit (r, j), B += 1, tau += a_{r,j};
     keep it while Theta = tau * SPS(B) beats Theta_best, stop at the first
     candidate that does not (the causal early stop)
  6. return the l_r that reached Theta_best.

Readings where the pages leave a choice (each one is also a design decision of
the GPU scheduler, which must agree bit for bit):
  * survival is the product of the fp32 confidences in float64, left to right;
  * a is quantised to Q50 fixed point, a_fx = floor(a * 2^50); a slot with
    a_fx = 0 is not a candidate (step 2's a > 0, at 2^-50 resolution).  tau is
    then an exact integer and the comparisons below are exact, so the result
    cannot depend on summation order;
  * Theta comparisons are exact (rational) products of the integer tau and the
    float64 table entry; an equal Theta stops the walk ("Theta > Theta_best,
    else break");
  * ties in a_fx go to the lower request, then the lower position (the pages
    favour the smaller request ID); the position rule keeps prefix closure
    when two consecutive survivals are equal;
  * the table must cover every batch the walk can reach: n_sps >= R (1 + gamma);
  * Theta_best is reported as float64: float(tau_fx) * 2^-50 * SPS(R + A),
    rounded in that order.

The production variant (DSpark reading notes, "adapting Algorithm 1 to real
hardware: two conflicts" and "the asynchronous fix, and why it stays
lossless"; paper-breakdown page, "engineering challenges in production",
inference paragraph): a stepped SPS curve can trap the early stop at a local
peak, and graph replay needs the verification batch before the current
round's confidences exist.  So the capacity K of round t is the optimum of a
walk with NO early stop over the confidences of round t - 2, and round t
fills exactly that many slots from its own, current ranking.  Readings:
  * the whole-walk optimum is the smallest m with the largest Theta(m),
    m = 0..M, compared exactly (an equal Theta does not buy more slots, as
    with the early stop's tie rule);
  * K counts admitted draft slots (A); the verification batch is R + K;
  * a round whose pool holds fewer than K candidates admits all M of them;
    K < 0 admits nothing;
  * rounds 0 and 1 have no confidences two rounds back: their capacity is
    given by the caller.
"""

from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np

Q = 50
ONE = 1 << Q


def survival(c: np.ndarray) -> np.ndarray:
    """a[r, j] = c[r, 0] * ... * c[r, j] in float64, multiplied left to right."""
    c64 = np.asarray(c, dtype=np.float32).astype(np.float64)
    R, gamma = c64.shape
    a = np.empty_like(c64)
    for r in range(R):
        s = 1.0
        for j in range(gamma):
            s = s * c64[r, j]
            a[r, j] = s
    return a


def quantise(a: np.ndarray) -> list:
    """a_fx = floor(a * 2^50) as Python ints (the scaling by 2^50 is exact)."""
    return [[int(math.floor(float(v) * float(ONE))) for v in row] for row in a]


def ranked_pool(c: np.ndarray) -> list:
    """Step 2: candidates (a_fx, r, j) with a_fx > 0, best first, ties to (r, j)."""
    afx = quantise(survival(c))
    pool = [(v, r, j) for r, row in enumerate(afx) for j, v in enumerate(row) if v > 0]
    pool.sort(key=lambda t: (-t[0], t[1], t[2]))
    return pool


def admit(c: np.ndarray, sps: np.ndarray) -> dict:
    """Algorithm 1 with the causal early stop, in exact arithmetic.

    c [R][gamma] fp32 conditional survivals; sps[B-1] = SPS(B).
    Returns ell [R] (admitted draft length), A = sum(ell), theta_best (float64),
    and the walk's trace for inspection."""
    c = np.asarray(c, dtype=np.float32)
    R, gamma = c.shape
    sps = np.asarray(sps, dtype=np.float64)
    if sps.shape[0] < R * (1 + gamma):
        raise ValueError("step-speed table shorter than R*(1+gamma)")
    pool = ranked_pool(c)
    tau = R * ONE
    B = R
    best = Fraction(tau) * Fraction(float(sps[B - 1]))
    ell = [0] * R
    A = 0
    trace = [(B, tau, best)]
    for v, r, j in pool:
        tau_new = tau + v
        B_new = B + 1
        theta = Fraction(tau_new) * Fraction(float(sps[B_new - 1]))
        trace.append((B_new, tau_new, theta))
        if theta > best:
            best, tau, B = theta, tau_new, B_new
            ell[r] = j + 1
            A += 1
        else:
            break
    theta_best = float(tau) * 2.0 ** -Q * float(sps[R + A - 1])
    return dict(ell=np.array(ell, dtype=np.int64), A=A, theta_best=theta_best,
                tau_fx=tau, pool=pool, trace=trace)


def admit_float(c: np.ndarray, sps: np.ndarray) -> dict:
    """Algorithm 1 exactly as the pages write it, in plain float64 (no
    quantisation, float accumulation of tau).  Used as a cross-check."""
    a = survival(c)
    R, gamma = a.shape
    pool = [(a[r, j], r, j) for r in range(R) for j in range(gamma) if a[r, j] > 0]
    pool.sort(key=lambda t: (-t[0], t[1], t[2]))
    tau, B = float(R), R
    best = tau * float(sps[B - 1])
    ell = [0] * R
    thetas = [best]
    for v, r, j in pool:
        tau_n, B_n = tau + v, B + 1
        theta = tau_n * float(sps[B_n - 1])
        thetas.append(theta)
        if theta > best:
            best, tau, B = theta, tau_n, B_n
            ell[r] = j + 1
        else:
            break
    return dict(ell=np.array(ell, dtype=np.int64), A=int(sum(ell)), theta_best=best,
                thetas=thetas)


def theta_curve(c: np.ndarray, sps: np.ndarray) -> list:
    """The whole walk without the early stop: [(B, tau*(B), Theta(B))] in float64,
    B = R .. R + |pool| (step 3 of the optimality sketch)."""
    a = survival(c)
    R, gamma = a.shape
    pool = sorted(((a[r, j], r, j) for r in range(R) for j in range(gamma) if a[r, j] > 0),
                  key=lambda t: (-t[0], t[1], t[2]))
    tau, B = float(R), R
    out = [(B, tau, tau * float(sps[B - 1]))]
    for v, r, j in pool:
        tau, B = tau + v, B + 1
        out.append((B, tau, tau * float(sps[B - 1])))
    return out


def admit_lookahead(c: np.ndarray, sps: np.ndarray) -> dict:
    """The walk WITHOUT the early stop: take the prefix that maximises Theta over
    the whole curve.  This is the look-ahead scheduler of Appendix A; it is not
    causal when later confidences depend on earlier draws."""
    a = survival(c)
    R, gamma = a.shape
    pool = sorted(((a[r, j], r, j) for r in range(R) for j in range(gamma) if a[r, j] > 0),
                  key=lambda t: (-t[0], t[1], t[2]))
    curve = theta_curve(c, sps)
    m_best = max(range(len(curve)), key=lambda m: (curve[m][2], -m))
    ell = [0] * R
    for v, r, j in pool[:m_best]:
        ell[r] = max(ell[r], j + 1)
    return dict(ell=np.array(ell, dtype=np.int64), A=m_best, theta_best=curve[m_best][2])


def brute_force_tau(c: np.ndarray, B: int) -> Fraction:
    """max over every length vector with sum(1 + l_r) = B of
    tau = sum_r (1 + sum_{j <= l_r} a_{r,j}), in exact arithmetic."""
    a = survival(c)
    R, gamma = a.shape
    best = None
    prefix = [[Fraction(0)] + list(itertools.accumulate(Fraction(float(v)) for v in a[r]))
              for r in range(R)]
    for ell in itertools.product(range(gamma + 1), repeat=R):
        if sum(1 + e for e in ell) != B:
            continue
        tau = sum(1 + prefix[r][ell[r]] for r in range(R))
        if best is None or tau > best:
            best = tau
    return best


def theta_walk_exact(c: np.ndarray, sps: np.ndarray) -> list:
    """The ranked walk in Q50 without the early stop: [(m, tau_fx(m), Theta(m))]
    for m = 0..M, Theta as an exact Fraction of the integer tau and the table
    entry (step 3 of the optimality sketch, in the scheduler's arithmetic)."""
    c = np.asarray(c, dtype=np.float32)
    R, gamma = c.shape
    sps = np.asarray(sps, dtype=np.float64)
    if sps.shape[0] < R * (1 + gamma):
        raise ValueError("step-speed table shorter than R*(1+gamma)")
    pool = ranked_pool(c)
    tau = R * ONE
    out = [(0, tau, Fraction(tau) * Fraction(float(sps[R - 1])))]
    for m, (v, r, j) in enumerate(pool, start=1):
        tau += v
        out.append((m, tau, Fraction(tau) * Fraction(float(sps[R + m - 1]))))
    return out


def _lengths_of_first(pool: list, A: int, R: int) -> np.ndarray:
    """l_r = one more than the largest position of request r among the first A
    ranked slots (the ranked prefix is prefix-closed per request, Lemma 1)."""
    ell = [0] * R
    for v, r, j in pool[:A]:
        ell[r] = max(ell[r], j + 1)
    return np.array(ell, dtype=np.int64)


def admit_full_scan(c: np.ndarray, sps: np.ndarray) -> dict:
    """The whole-walk optimum: A = the smallest m maximising Theta(m) over
    m = 0..M.  Run on the confidences of round t - 2, its A is the capacity K
    of round t."""
    c = np.asarray(c, dtype=np.float32)
    R = c.shape[0]
    walk = theta_walk_exact(c, sps)
    best_m, best_tau, best_theta = walk[0]
    for m, tau, theta in walk[1:]:
        if theta > best_theta:
            best_m, best_tau, best_theta = m, tau, theta
    pool = ranked_pool(c)
    theta_best = float(best_tau) * 2.0 ** -Q * float(np.asarray(sps, dtype=np.float64)[R + best_m - 1])
    return dict(ell=_lengths_of_first(pool, best_m, R), A=best_m, theta_best=theta_best, tau_fx=best_tau)


def admit_capacity(c: np.ndarray, sps: np.ndarray, K: int) -> dict:
    """Fill a capacity of K draft slots from the current ranking: the first
    min(max(K, 0), M) ranked slots are admitted, whatever Theta does."""
    c = np.asarray(c, dtype=np.float32)
    R = c.shape[0]
    walk = theta_walk_exact(c, sps)
    M = len(walk) - 1
    A = min(max(int(K), 0), M)
    _, tau, _ = walk[A]
    theta_best = float(tau) * 2.0 ** -Q * float(np.asarray(sps, dtype=np.float64)[R + A - 1])
    return dict(ell=_lengths_of_first(ranked_pool(c), A, R), A=A, theta_best=theta_best, tau_fx=tau)


def production_schedule(c_rounds: list, sps: np.ndarray, K_init: int) -> list:
    """The asynchronous scheduler over a sequence of rounds: round t admits
    with capacity K_t = admit_full_scan(c_{t-2}).A (K_init for t = 0, 1)."""
    out = []
    for t, c in enumerate(c_rounds):
        K = K_init if t < 2 else admit_full_scan(c_rounds[t - 2], sps)["A"]
        res = admit_capacity(c, sps, K)
        res["K"] = K
        out.append(res)
    return out
