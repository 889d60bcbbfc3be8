"""One draft-and-verify round, free running, in the order of the end-to-end loop
(DSpark reading notes, "full decode loop" pseudocode steps 3-13; caijizhuo
page, dspark_cycle steps 3-6): sample the gamma-block, score it with the
confidence head, schedule the batch, verify the admitted prefixes.

The inputs are the stored arrays of a workload (bf16 bits or fp32) and are
upcast exactly to float64 here.  `requests` restricts the per-request stages
(sampling, confidence, verification) to a subset, which is how a bounded
sample of a large workload is timed; the scheduler then ranks the subset's
slots only."""

from __future__ import annotations

import numpy as np

from .common import as_f64
from .confidence import confidence
from .sample import markov_sample
from .schedule import admit
from .verify import verify


def run_round(inp, requests=None) -> dict:
    dt = inp.w.dtype
    idx = np.arange(inp.w.R) if requests is None else np.asarray(requests)
    U = as_f64(inp.U[idx], dt)
    E = as_f64(inp.E, dt)
    W2t = as_f64(inp.W2t, dt)
    x0 = inp.x0[idx].astype(np.int64)
    s = markov_sample(U, E, W2t, x0, inp.G_by_request(idx), inp.g[idx])
    cf = confidence(as_f64(inp.h[idx], dt), as_f64(inp.w_conf, dt), E, x0, s["x"], inp.T)
    sc = admit(cf["c"].astype(np.float32), inp.sps)
    ell = sc["ell"]
    tgt = as_f64(inp.target[idx], dt)
    vf = verify(tgt, None, U, E, W2t, x0, s["x"], ell, inp.u_acc[idx], inp.u_res[idx])
    return dict(x=s["x"], lse=s["lse"], logit=s["logit"], z=cf["z"], c=cf["c"],
                ell=ell, A=sc["A"], theta_best=sc["theta_best"],
                n_acc=vf["n_acc"], next_tok=vf["next_tok"])
