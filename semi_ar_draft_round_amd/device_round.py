"""One draft-and-verify round on the GPU through the C ABI.

`to_device` copies a RoundInputs (the seeded arrays of workloads.py) into
device tensors once, with every output buffer and workspace preallocated, so
that `run_round` only enqueues its three library calls and can be captured in
a HIP graph.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import binding as B


def _dev_store(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


@dataclasses.dataclass
class DeviceRound:
    R: int
    gamma: int
    V: int
    r: int
    d: int
    U: torch.Tensor
    W1: torch.Tensor
    W2t: torch.Tensor
    w: torch.Tensor
    h: torch.Tensor
    x0: torch.Tensor
    target: Optional[torch.Tensor]
    sps: torch.Tensor
    T: Optional[torch.Tensor]
    G: torch.Tensor
    g: torch.Tensor
    u_acc: torch.Tensor
    u_res: torch.Tensor
    # outputs
    x: torch.Tensor
    lse: torch.Tensor
    logit: torch.Tensor
    c: torch.Tensor
    z: torch.Tensor
    ell: torch.Tensor
    admitted: torch.Tensor
    theta_best: torch.Tensor
    n_acc: torch.Tensor
    next_tok: torch.Tensor
    ws_sample: torch.Tensor
    ws_sched: torch.Tensor
    ws_verify: torch.Tensor
    status: torch.Tensor
    # the production scheduler: this round's capacity, its fill, and the
    # capacity its confidences set for two rounds later
    cap: torch.Tensor
    ell_p: torch.Tensor
    admitted_p: torch.Tensor
    theta_p: torch.Tensor
    cap_next: torch.Tensor
    ell_w: torch.Tensor
    theta_w: torch.Tensor
    # greedy verification and the analytic acceptance
    n_acc_g: torch.Tensor
    next_tok_g: torch.Tensor
    c_star: torch.Tensor
    ws_greedy: torch.Tensor
    ws_accept: torch.Tensor
    # sampling with the RNN head (allocated when asked for)
    rnn: Optional[dict] = None


def to_device(inp, device="cuda:0", rnn: bool = False) -> DeviceRound:
    w = inp.w
    dev = torch.device(device)
    R, gamma, V, r, d = w.R, w.gamma, w.V, w.r, w.d
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    dr = DeviceRound(
        R, gamma, V, r, d,
        U=_dev_store(inp.U, w.dtype, dev), W1=_dev_store(inp.E, w.dtype, dev),
        W2t=_dev_store(inp.W2t, w.dtype, dev), w=_dev_store(inp.w_conf, w.dtype, dev),
        h=_dev_store(inp.h, w.dtype, dev), x0=i32(inp.x0),
        target=None if inp.target is None else _dev_store(inp.target, w.dtype, dev),
        sps=torch.from_numpy(np.ascontiguousarray(inp.sps, dtype=np.float64)).to(dev),
        T=None if inp.T is None else f32(inp.T),
        G=f32(inp.G), g=f32(inp.g), u_acc=f32(inp.u_acc), u_res=f32(inp.u_res),
        x=torch.empty((R, gamma), dtype=torch.int32, device=dev),
        lse=torch.empty((R, gamma), dtype=torch.float32, device=dev),
        logit=torch.empty((R, gamma), dtype=torch.float32, device=dev),
        c=torch.empty((R, gamma), dtype=torch.float32, device=dev),
        z=torch.empty((R, gamma), dtype=torch.float32, device=dev),
        ell=torch.empty(R, dtype=torch.int32, device=dev),
        admitted=torch.empty(1, dtype=torch.int32, device=dev),
        theta_best=torch.empty(1, dtype=torch.float64, device=dev),
        n_acc=torch.empty(R, dtype=torch.int32, device=dev),
        next_tok=torch.empty(R, dtype=torch.int32, device=dev),
        ws_sample=torch.empty(max(1, B.dspark_workspace_size(B.WS_SAMPLE, R, gamma, V, r)),
                              dtype=torch.uint8, device=dev),
        ws_sched=torch.empty(max(1, B.dspark_workspace_size(B.WS_SCHEDULE, R, gamma, V, r)),
                             dtype=torch.uint8, device=dev),
        ws_verify=torch.empty(max(1, B.dspark_workspace_size(B.WS_VERIFY, R, gamma, V, r)),
                              dtype=torch.uint8, device=dev),
        status=torch.zeros(1, dtype=torch.int32, device=dev),
        cap=torch.full((1,), R * gamma // 8, dtype=torch.int32, device=dev),
        ell_p=torch.empty(R, dtype=torch.int32, device=dev),
        admitted_p=torch.empty(1, dtype=torch.int32, device=dev),
        theta_p=torch.empty(1, dtype=torch.float64, device=dev),
        cap_next=torch.empty(1, dtype=torch.int32, device=dev),
        ell_w=torch.empty(R, dtype=torch.int32, device=dev),
        theta_w=torch.empty(1, dtype=torch.float64, device=dev),
        n_acc_g=torch.empty(R, dtype=torch.int32, device=dev),
        next_tok_g=torch.empty(R, dtype=torch.int32, device=dev),
        c_star=torch.empty((R, gamma), dtype=torch.float32, device=dev),
        ws_greedy=torch.empty(max(1, B.dspark_workspace_size(B.WS_VERIFY_GREEDY, R, gamma, V, r)),
                              dtype=torch.uint8, device=dev),
        ws_accept=torch.empty(max(1, B.dspark_workspace_size(B.WS_ACCEPTANCE, R, gamma, V, r)),
                              dtype=torch.uint8, device=dev),
    )
    if rnn:
        from .workloads import make_rnn_weights
        dr.rnn = dict(
            W=_dev_store(make_rnn_weights(w), w.dtype, dev),
            x=torch.empty((R, gamma), dtype=torch.int32, device=dev),
            lse=torch.empty((R, gamma), dtype=torch.float32, device=dev),
            logit=torch.empty((R, gamma), dtype=torch.float32, device=dev),
            s=torch.empty((R, gamma, r), dtype=torch.float32, device=dev),
            o=torch.empty((R, gamma, r), dtype=dr.U.dtype, device=dev),
            ws=torch.empty(max(1, B.dspark_workspace_size(B.WS_RNN_SAMPLE, R, gamma, V, r)),
                           dtype=torch.uint8, device=dev),
        )
    return dr


def sample(d: DeviceRound):
    B.dspark_markov_sample(d.U, d.W1, d.W2t, d.x0, d.G, d.g, d.x, d.lse, d.logit, ws=d.ws_sample)


def sample_conf(d: DeviceRound, timer=None):
    """The draft and its confidences in one call (dspark_markov_sample_ex):
    the sampler's finalize step scores every position.  timer: a
    binding.SweepTimer to stamp with the position sweep (eager calls only)."""
    B.dspark_markov_sample_ex(d.U, d.W1, d.W2t, d.x0, d.G, d.g, h=d.h, w=d.w, T=d.T, x=d.x, lse=d.lse,
                              logit=d.logit, c=d.c, z=d.z, status=d.status, ws=d.ws_sample, timer=timer)


def confidence(d: DeviceRound):
    B.dspark_confidence(d.h, d.w, d.W1, d.x0, d.x, d.T, d.c, d.z)


def schedule(d: DeviceRound):
    B.dspark_schedule(d.c, d.sps, d.ell, d.admitted, d.theta_best, ws=d.ws_sched)


def schedule_production(d: DeviceRound):
    """The asynchronous scheduler's two calls: fill this round's capacity
    from the current ranking, then the whole-walk optimum of the current
    confidences, which is the capacity two rounds later."""
    B.dspark_schedule_ex(d.c, d.sps, B.SCHED_CAPACITY, d.cap, d.ell_p, d.admitted_p, d.theta_p, ws=d.ws_sched)
    B.dspark_schedule_ex(d.c, d.sps, B.SCHED_WHOLE_WALK, None, d.ell_w, d.cap_next, d.theta_w, ws=d.ws_sched)


def rnn_sample(d: DeviceRound):
    """The round's draft with the RNN head instead of the Markov head."""
    q = d.rnn
    B.dspark_rnn_sample(d.U, d.W1, d.W2t, q["W"], d.h, d.x0, d.G, d.g, q["x"], q["lse"], q["logit"], q["s"],
                        q["o"], q["ws"], P=q.get("P"))


def rnn_prepare(d: DeviceRound):
    """The W1-row part of the RNN head's projection for every token, kept
    with the round's RNN weights (bf16; done once per set of weights)."""
    d.rnn["P"] = B.dspark_rnn_prepare(d.W1, d.rnn["W"], d.h.shape[2], P=d.rnn.get("P"))


def verify_greedy(d: DeviceRound):
    """Temperature-0 verification of the round's drafts and admitted lengths."""
    B.dspark_verify_greedy(d.target, d.x, d.ell, n_acc=d.n_acc_g, next_tok=d.next_tok_g, ws=d.ws_greedy)


def acceptance(d: DeviceRound):
    """The analytic acceptance of every drafted position of the round."""
    B.dspark_acceptance(d.target, d.U, d.W1, d.W2t, d.x0, d.x, d.lse, c_star=d.c_star, ws=d.ws_accept)


def verify(d: DeviceRound):
    B.dspark_verify(d.target, d.U, d.W1, d.W2t, d.x0, d.x, d.lse, d.logit, d.ell, d.u_acc,
                    d.u_res, n_acc=d.n_acc, next_tok=d.next_tok, ws=d.ws_verify)


def run_round(d: DeviceRound):
    """Enqueue one round on the current stream: the draft with its
    confidences (one call), the schedule, the verification."""
    sample_conf(d)
    schedule(d)
    verify(d)


def run_round_four_calls(d: DeviceRound):
    """The same round as the four separate calls sample -> confidence ->
    schedule -> verify."""
    sample(d)
    confidence(d)
    schedule(d)
    verify(d)


def outputs_to_host(d: DeviceRound) -> dict:
    torch.cuda.synchronize()
    return dict(x=d.x.cpu().numpy(), lse=d.lse.cpu().numpy(), logit=d.logit.cpu().numpy(),
                c=d.c.cpu().numpy(), z=d.z.cpu().numpy(), ell=d.ell.cpu().numpy(),
                A=int(d.admitted.cpu()[0]), theta_best=float(d.theta_best.cpu()[0]),
                n_acc=d.n_acc.cpu().numpy(), next_tok=d.next_tok.cpu().numpy())
