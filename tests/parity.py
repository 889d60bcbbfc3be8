"""Parity rules between the HIP path's outputs and the float64 oracle.

The oracle is teacher-forced on the GPU's own decisions (the previous token
at each position, the confidences fed to the scheduler, the admitted
lengths and the accepted lengths fed to the residual draw), so that one
tolerated near-tie cannot cascade into later mismatches.

Tolerances:
  tokens     equal to the oracle's two-level Gumbel-max draw, or within a
             perturbed-score gap of 1e-4 at both levels
  lse        1e-5 relative (of max(1, |lse|))
  logit      1e-5 of max(1, |logit|)
  c          1e-5 relative; z 1e-5 of max(1, |z|)
  schedule   ell, A and theta_best bit-exact
  n_acc      exact, except where |ln u - ln ratio| <= 1e-5 (near-tie)
  next_tok   equal to the oracle's inverse-CDF draw, or u_res within the
             row's CDF bound of the GPU token's CDF interval, and at most one
             such token per check.  The bound is 1e-6 (the fp32 scan over the
             chunk masses) plus what the GPU's fp32 draft and target logits
             can move the normalised residual: each logit within
             LOGIT_FP32 * max(1, |l|) of the exact one changes p_d(v) and
             p_t(v) by at most a factor exp(2 * that), so r(v) = max(0, p_t -
             p_d) by at most their sum, and the normalised CDF by at most
             twice the sum of those changes over Z = sum of r
"""

from __future__ import annotations

import numpy as np

from oracle.common import as_f64
from oracle.confidence import confidence as oracle_confidence
from oracle.sample import markov_sample, token_gaps
from oracle.schedule import admit
from oracle import verify as OV

TOK_GAP = 1e-4
LSE_REL = 1e-5
LOGIT_TOL = 1e-5
C_REL = 1e-5
Z_TOL = 1e-5
ACC_TIE = 1e-5
CDF_TOL = 1e-6
MAX_TOK_TOL = 1   # tokens per check allowed inside the CDF tolerance band
LOGIT_FP32 = 1e-6   # error of a GPU logit (fp32 bias accumulation onto the stored logit), of max(1, |l|)


def residual_cdf_bound(tgt, r0, U, E, W2t, x0, x, i, n, ell_i):
    """How far the GPU's normalised residual CDF can sit from the oracle's
    for request i with n accepted drafts (see the module docstring)."""
    lt = OV._target_row(tgt, r0, i, n)
    pt = np.exp(lt - np.logaddexp.reduce(lt))
    dt = np.expm1(2.0 * LOGIT_FP32 * np.maximum(1.0, np.abs(lt)))
    if n >= ell_i:                                   # bonus row: p_t itself
        return CDF_TOL + 2.0 * float((pt * dt).sum())
    ld = OV.draft_logits_at(U, E, W2t, x0, x, i, n)
    pd = np.exp(ld - np.logaddexp.reduce(ld))
    Z = float(np.maximum(0.0, pt - pd).sum())
    if not Z > 0.0:
        return CDF_TOL
    dd = np.expm1(2.0 * LOGIT_FP32 * np.maximum(1.0, np.abs(ld)))
    return CDF_TOL + 2.0 * float((pt * dt + pd * dd).sum()) / Z


def check_sample(inp, gpu, idx):
    """Teacher-forced sampling parity on requests idx.  Returns a report."""
    dt = inp.w.dtype
    U = as_f64(inp.U[idx], dt)
    E = as_f64(inp.E, dt)
    W2t = as_f64(inp.W2t, dt)
    xg = gpu["x"][idx].astype(np.int64)
    out = markov_sample(U, E, W2t, inp.x0[idx].astype(np.int64), inp.G_by_request(idx), inp.g[idx],
                        teacher_x=xg, keep_steps=True)
    gamma = U.shape[1]
    worst = dict(chunk_gap=0.0, inner_gap=0.0, lse=0.0, logit=0.0, exact=0, total=0)
    assert xg.min() >= 0 and xg.max() < inp.w.V, "token out of range"
    for k in range(gamma):
        st = out["steps"][k]
        cg, ig = token_gaps(st, inp.g[idx][:, k, :], xg[:, k])
        worst["chunk_gap"] = max(worst["chunk_gap"], float(cg.max()))
        worst["inner_gap"] = max(worst["inner_gap"], float(ig.max()))
        worst["exact"] += int(np.sum(st["token"] == xg[:, k]))
        worst["total"] += len(idx)
        lse_err = np.abs(gpu["lse"][idx, k] - st["lse"]) / np.maximum(1.0, np.abs(st["lse"]))
        worst["lse"] = max(worst["lse"], float(lse_err.max()))
        lg = st["l"][np.arange(len(idx)), xg[:, k]]
        lg_err = np.abs(gpu["logit"][idx, k] - lg) / np.maximum(1.0, np.abs(lg))
        worst["logit"] = max(worst["logit"], float(lg_err.max()))
    assert worst["chunk_gap"] <= TOK_GAP, worst
    assert worst["inner_gap"] <= TOK_GAP, worst
    assert worst["lse"] <= LSE_REL, worst
    assert worst["logit"] <= LOGIT_TOL, worst
    return worst


def check_confidence(inp, gpu, idx):
    dt = inp.w.dtype
    ref = oracle_confidence(as_f64(inp.h[idx], dt), as_f64(inp.w_conf, dt), as_f64(inp.E, dt),
                            inp.x0[idx].astype(np.int64), gpu["x"][idx].astype(np.int64), inp.T)
    c_err = np.abs(gpu["c"][idx] - ref["c"]) / np.maximum(ref["c"], 1e-300)
    z_err = np.abs(gpu["z"][idx] - ref["z"]) / np.maximum(1.0, np.abs(ref["z"]))
    rep = dict(c=float(c_err.max()), z=float(z_err.max()))
    assert rep["c"] <= C_REL, rep
    assert rep["z"] <= Z_TOL, rep
    return rep


def check_schedule(inp_sps, gpu):
    """Bit-exact scheduler parity on the GPU's confidences (whole batch)."""
    ref = admit(gpu["c"].astype(np.float32), inp_sps)
    assert gpu["ell"].tolist() == ref["ell"].tolist(), (gpu["ell"], ref["ell"])
    assert gpu["A"] == ref["A"]
    assert gpu["theta_best"] == ref["theta_best"], (gpu["theta_best"], ref["theta_best"])
    return dict(A=ref["A"])


def check_verify(inp, gpu, idx, target=None, row0=None):
    dt = inp.w.dtype
    U = as_f64(inp.U[idx], dt)
    E = as_f64(inp.E, dt)
    W2t = as_f64(inp.W2t, dt)
    x0 = inp.x0[idx].astype(np.int64)
    x = gpu["x"][idx].astype(np.int64)
    ell = gpu["ell"][idx].astype(np.int64)
    n_gpu = gpu["n_acc"][idx].astype(np.int64)
    if target is None:
        tgt = as_f64(inp.target[idx], dt)
        r0 = None
    else:
        tgt, r0 = target, row0
    u_acc = inp.u_acc[idx]
    logr = OV.accept_log_ratios(tgt, r0, U, E, W2t, x0, x, ell)
    rep = dict(n_exact=0, n_ties=0, tok_exact=0, tok_tol=0, total=len(idx))
    for i in range(len(idx)):
        lr = logr[i]
        lu = np.log(u_acc[i, :len(lr)].astype(np.float64))
        n_or = OV.first_rejection(lr, u_acc[i])
        ng = int(n_gpu[i])
        assert 0 <= ng <= ell[i]
        # the GPU accepted every p < ng and rejected ng (if ng < ell); each
        # decision must agree with the oracle's or be a near-tie
        for p in range(min(ng + 1, len(lr))):
            acc_gpu = p < ng
            acc_or = bool(lu[p] < lr[p])
            if acc_or != acc_gpu:
                assert abs(lu[p] - lr[p]) <= ACC_TIE, (i, p, lu[p], lr[p])
                rep["n_ties"] += 1
        rep["n_exact"] += int(ng == n_or)
        res = OV.residual(tgt, r0, U, E, W2t, x0, x, i, ng, int(ell[i]))
        tok = int(gpu["next_tok"][idx[i]])
        assert 0 <= tok < inp.w.V
        want = OV.inverse_cdf(res, float(inp.u_res[idx[i]]))
        if tok == want:
            rep["tok_exact"] += 1
        else:
            lo, hi = OV.cdf_interval(res, tok)
            u = float(inp.u_res[idx[i]])
            tol = residual_cdf_bound(tgt, r0, U, E, W2t, x0, x, i, ng, int(ell[i]))
            assert lo - tol <= u <= hi + tol, (i, tok, want, lo, hi, u, tol)
            rep["tok_tol"] += 1
    assert rep["tok_tol"] <= MAX_TOK_TOL, rep
    return rep


def gpu_outputs_subset_ok(gpu, R, gamma):
    assert gpu["x"].shape == (R, gamma)
    assert np.all(np.isfinite(gpu["lse"])) and np.all(np.isfinite(gpu["c"]))
