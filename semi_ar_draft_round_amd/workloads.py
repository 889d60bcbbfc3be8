"""Seeded synthetic inputs for one draft-and-verify round.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic.  Both the HIP path and the CPU oracle read the exact
arrays it returns (the same bf16 / fp32 bits), so any difference between the
two comes from the computation, never from the data.

Value distributions follow the workloads the DSpark pages describe for the
drafter (arXiv:2607.05147): base logits with a peaked token on half of the
positions, a rank-256 Markov head, a linear confidence head, a target model
whose logits are a noisy copy of the drafter's, and a step-speed table that
does not increase with the batch size.  The second argument of N(., .) is a
variance throughout (the pages write the logit spread as N(0, 2^2)).

Random draws that the method itself makes are inputs too:
  G     [gamma][nC][R]  one Gumbel per 16-token chunk of the vocabulary, per
                        position and request (request-minor, the layout the
                        library reads),
  g     [R][gamma][16]  the in-chunk Gumbels, shared by every chunk,
  u_acc [R][gamma]      one uniform per drafted position for the accept test,
  u_res [R]             one uniform per request for the residual / bonus draw.
Uniforms are odd multiples of 2^-24, so they lie strictly inside (0, 1) and
are exact in fp32; a Gumbel is -ln(-ln u) evaluated in fp64 and rounded once
to fp32.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CHUNK = 16  # tokens per chunk of the two-level Gumbel draw (shape of G and g)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    R: int
    gamma: int
    V: int
    r: int
    d: int
    dtype: str                 # "f32" or "bf16": storage type of U, E, W2t, w, h, target
    spike: str                 # "const6" or "uniform8"
    target_sigma: str          # "one" or "uniform0.5-2"
    sps: str                   # step-speed table recipe
    temperatures: bool         # per-position temperatures T_k in [1, 2]
    seed: int

    @property
    def n_chunks(self) -> int:
        return (self.V + CHUNK - 1) // CHUNK

    @property
    def n_sps(self) -> int:
        return len(make_sps(self))


# The five synthetic workloads.  The first is small enough for the oracle to
# run whole in seconds; the fourth is the one the throughput is quoted on.
WORKLOADS = [
    Workload("tiny_r1_g4_v1024_f32", 1, 4, 1024, 32, 64, "f32",
             "const6", "one", "rand8", False, 20260000),
    Workload("latency_r1_g16_v151936", 1, 16, 151936, 256, 4096, "bf16",
             "const6", "one", "stair_17", False, 20260100),
    Workload("batch_r32_g16_v151936", 32, 16, 151936, 256, 4096, "bf16",
             "uniform8", "one", "stair_4096", False, 20260200),
    Workload("heavy_r128_g16_v129280", 128, 16, 129280, 256, 7168, "bf16",
             "uniform8", "uniform0.5-2", "hyper_4096", False, 20260300),
    Workload("full_r256_g16_v129280_sts", 256, 16, 129280, 256, 7168, "bf16",
             "uniform8", "uniform0.5-2", "hyper_4352", True, 20260400),
]
BY_NAME = {w.name: w for w in WORKLOADS}
BENCH_WORKLOAD = "heavy_r128_g16_v129280"


def custom(name: str, R: int, gamma: int, V: int, r: int, d: int, dtype: str = "bf16",
           seed: int = 1234, spike: str = "uniform8", target_sigma: str = "uniform0.5-2",
           sps: str = "hyper_auto", temperatures: bool = False) -> Workload:
    """A workload of arbitrary size drawn with the same recipe."""
    return Workload(name, R, gamma, V, r, d, dtype, spike, target_sigma, sps, temperatures, seed)


# ---------------------------------------------------------------- helpers

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    out = ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def _stored_f32(stored: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_to_f32(stored) if dtype == "bf16" else stored


def odd_uniform(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniforms (2k+1)/2^24, k uniform in [0, 2^23): exact in fp32, inside (0, 1)."""
    k = rng.integers(0, 1 << 23, size=shape, dtype=np.int64)
    return ((2 * k + 1).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def gumbel_from_uniform(u: np.ndarray) -> np.ndarray:
    u64 = u.astype(np.float64)
    return (-np.log(-np.log(u64))).astype(np.float32)


def make_sps(w: Workload) -> np.ndarray:
    """Step-speed table, sps[B-1] = SPS(B) in steps/s, non-increasing in B."""
    kind = w.sps
    if kind == "rand8":
        rng = np.random.default_rng(w.seed + 7)
        vals = np.sort(rng.integers(100, 1001, size=8))[::-1]
        return vals.astype(np.float64).copy()

    def stair(B):  # 1000 up to B=64, then 1000/(1+(B-64)/256), floored to a multiple of 8
        return 8.0 * np.floor(1000.0 / (1.0 + np.maximum(0, B - 64) / 256.0) / 8.0)

    def hyper(B):  # integer-stepped 4096000/(B+2048)
        return np.floor(4096000.0 / (B + 2048.0))

    if kind.startswith("stair_"):
        n = int(kind.split("_")[1])
        return stair(np.arange(1, n + 1, dtype=np.float64))
    if kind.startswith("hyper_"):
        tail = kind.split("_")[1]
        n = w.R * (1 + w.gamma) if tail == "auto" else int(tail)
        return hyper(np.arange(1, n + 1, dtype=np.float64))
    raise ValueError(kind)


@dataclasses.dataclass
class RoundInputs:
    w: Workload
    U: np.ndarray          # [R][gamma][V]   bf16 bits (uint16) or float32
    E: np.ndarray          # [V][r]          W1, token -> r-vector
    W2t: np.ndarray        # [V][r]          W2 stored transposed: row v is column v of W2
    w_conf: np.ndarray     # [d + r]         confidence weights, h-part then W1-part
    h: np.ndarray          # [R][gamma][d]   backbone hidden states
    x0: np.ndarray         # [R] int32       anchors
    target: np.ndarray     # [R][gamma+1][V] target logits; row i predicts draft position i
    sps: np.ndarray        # [n_sps] float64
    T: Optional[np.ndarray]  # [gamma] float32 or None
    G: np.ndarray          # [gamma][nC][R] float32
    g: np.ndarray          # [R][gamma][CHUNK] float32
    u_acc: np.ndarray      # [R][gamma] float32
    u_res: np.ndarray      # [R] float32

    @property
    def dtype(self) -> str:
        return self.w.dtype

    def G_by_request(self, idx=None) -> np.ndarray:
        """G as [R][gamma][nC] (a transposed view), optionally for requests idx."""
        Gr = np.transpose(self.G, (2, 0, 1))
        return Gr if idx is None else Gr[idx]


def make_inputs(w: Workload, round_index: int = 0, with_target: bool = True) -> RoundInputs:
    """Draw one round of inputs.  Weights depend on the workload seed only;
    per-round data (logits, hidden states, anchors, noise) also on round_index."""
    R, gamma, V, r, d = w.R, w.gamma, w.V, w.r, w.d
    wrng = np.random.default_rng([w.seed, 0])
    rng = np.random.default_rng([w.seed, 1 + round_index])

    E = _store(wrng.standard_normal((V, r), dtype=np.float32) * np.float32(math.sqrt(0.02)), w.dtype)
    W2t = _store(wrng.standard_normal((V, r), dtype=np.float32) * np.float32(math.sqrt(1.0 / r)), w.dtype)
    w_conf = _store(wrng.standard_normal(d + r, dtype=np.float32) * np.float32(math.sqrt(0.05)), w.dtype)

    # base logits: N(0, 4), plus a spike on one uniform token at half of the positions
    U32 = rng.standard_normal((R, gamma, V), dtype=np.float32)
    U32 *= np.float32(2.0)
    n_spike = (R * gamma) // 2
    pos = rng.permutation(R * gamma)[:n_spike]
    tok = rng.integers(0, V, size=n_spike)
    if w.spike == "const6":
        mag = np.full(n_spike, 6.0, dtype=np.float32)
    else:
        m_r = rng.uniform(0.0, 8.0, size=R).astype(np.float32)
        mag = m_r[pos // gamma]
    U32.reshape(R * gamma, V)[pos, tok] += mag
    U = _store(U32, w.dtype)
    del U32

    h = _store(rng.standard_normal((R, gamma, d), dtype=np.float32), w.dtype)
    x0 = rng.integers(0, V, size=R).astype(np.int32)

    if w.target_sigma == "one":
        sigma = np.ones(R, dtype=np.float32)
    else:
        sigma = rng.uniform(0.5, 2.0, size=R).astype(np.float32)

    target = None
    if with_target:
        t32 = np.empty((R, gamma + 1, V), dtype=np.float32)
        t32[:, :gamma, :] = _stored_f32(U, w.dtype)
        fresh = rng.standard_normal((R, V), dtype=np.float32) * np.float32(2.0)
        ftok = rng.integers(0, V, size=R)
        fresh[np.arange(R), ftok] += np.float32(6.0)
        t32[:, gamma, :] = fresh
        del fresh
        for rr in range(R):  # per-request noise level, row by row to bound memory
            t32[rr] += rng.standard_normal((gamma + 1, V), dtype=np.float32) * sigma[rr]
        target = _store(t32, w.dtype)
        del t32

    sps = make_sps(w)
    T = None
    if w.temperatures:
        k = np.arange(gamma, dtype=np.float64)
        T = (1.0 + k / max(1, gamma - 1)).astype(np.float32)

    nC = w.n_chunks
    G = gumbel_from_uniform(odd_uniform(rng, (gamma, nC, R)))
    g = gumbel_from_uniform(odd_uniform(rng, (R, gamma, CHUNK)))
    u_acc = odd_uniform(rng, (R, gamma))
    u_res = odd_uniform(rng, (R,))
    return RoundInputs(w, U, E, W2t, w_conf, h, x0, target, sps, T, G, g, u_acc, u_res)


def make_rnn_weights(w: Workload, gain: float = 1.0) -> np.ndarray:
    """The RNN head's packed projection [3r][2r + d] (gate, candidate and
    output rows; columns state, W1 row, hidden state), N(0, gain^2 / (2r + d)),
    in the workload's storage type.  Seeded by the workload only."""
    rng = np.random.default_rng([w.seed, 7])
    K = 2 * w.r + w.d
    W = rng.normal(0.0, gain / np.sqrt(K), size=(3 * w.r, K)).astype(np.float32)
    return _store(W, w.dtype)


def make_rollouts(N: int, gamma: int, beta: float = 2.0, seed: int = 99):
    """A synthetic held-out set for calibrating the confidence head: each
    rollout's true conditional acceptance at position k is q ~ Beta(6, 2);
    the head reports the logit z = beta * logit(q) (beta > 1: overconfident);
    the rollout accepts position k with probability q_k until its first
    rejection.  Returns z [N][gamma] float32 and n_acc [N] int32 (0..gamma)."""
    rng = np.random.default_rng([seed, N, gamma])
    q = rng.beta(6.0, 2.0, size=(N, gamma))
    z = (np.log(q / (1.0 - q)) * beta).astype(np.float32)
    acc = rng.random((N, gamma)) < q
    n_acc = np.where(acc.all(axis=1), gamma, np.argmin(acc, axis=1)).astype(np.int32)
    return z, n_acc


def sts_grid(G: int = 61, lo: float = 0.25, hi: float = 8.0) -> np.ndarray:
    """Log-spaced candidate temperatures, with T = 1 itself when the range
    holds it at a grid point."""
    g = np.exp(np.linspace(np.log(lo), np.log(hi), G)).astype(np.float32)
    i = int(np.argmin(np.abs(np.log(g))))
    if abs(np.log(g[i])) < 1e-6:
        g[i] = 1.0
    return g

