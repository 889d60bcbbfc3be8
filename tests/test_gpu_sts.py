"""GPU sequential temperature scaling (dspark_sts_fit) against the oracle,
teacher-forced on the GPU's chosen temperatures.

ECE_TOL: predictions are fp32 on both sides, but the GPU's and numpy's
exp may differ in the last place (about 1.2e-7 relative on p), which moves
a bin sum by at most N * 1.2e-7 and the ECE by 1.2e-7; a prediction that
sits within that distance of a bin edge can land in the neighbouring bin,
moving the ECE by at most 2/N.  ECE_TOL = 2.5/N + 1e-6.  A chosen
temperature must be the oracle's, or one whose oracle ECE is within ECE_TOL
of the oracle's minimum.  The AUC is an exact pair count on the same fp32
logits on both sides: equal to 1e-12."""

import sys

import numpy as np
import pytest

from oracle import sts as OS
from semi_ar_draft_round_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from semi_ar_draft_round_amd import binding
    binding.load_library()
    return torch.device("cuda:0")


def _run(z, n_acc, grid, M, dev):
    from semi_ar_draft_round_amd import binding as B
    out = B.dspark_sts_fit(torch.tensor(z, device=dev), torch.tensor(n_acc, device=dev),
                           torch.tensor(grid, device=dev), M)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


@pytest.mark.parametrize("N,gamma,beta,M", [(20000, 4, 2.0, 15), (5000, 6, 1.0, 10), (777, 3, 3.0, 15),
                                           (65536, 16, 2.0, 15), (20000, 64, 2.0, 15)])
def test_sts_matches_oracle(N, gamma, beta, M, dev):
    say(f"[sts] N={N} gamma={gamma} beta={beta} M={M}")
    z, n_acc = W.make_rollouts(N, gamma, beta)
    grid = W.sts_grid()
    T, e0, e1, auc = _run(z, n_acc, grid, M, dev)
    ref = OS.sts_fit(z, n_acc, grid, M, teacher_T=T)
    tol = 2.5 / N + 1e-6
    for k in range(gamma):
        t = int(np.flatnonzero(grid == T[k])[0])
        assert ref["ece_grid"][k, t] <= ref["ece_grid"][k].min() + tol, k
        assert abs(e1[k] - ref["ece_grid"][k, t]) <= tol, (k, e1[k], ref["ece_grid"][k, t])
        assert abs(e0[k] - ref["ece_before"][k]) <= tol, (k, e0[k], ref["ece_before"][k])
        if np.isnan(ref["auc"][k]):
            assert np.isnan(auc[k])
        else:
            assert abs(auc[k] - ref["auc"][k]) <= 1e-12, (k, auc[k], ref["auc"][k])
    say(f"  T {T.round(3).tolist()}\n  ece {np.round(e0, 4).tolist()} -> {np.round(e1, 4).tolist()}\n"
        f"  auc {np.round(auc, 4).tolist()}")
    if beta > 1:
        assert np.all(e1 < e0)


def test_sts_is_deterministic(dev):
    z, n_acc = W.make_rollouts(30000, 5, 2.0)
    grid = W.sts_grid()
    a = _run(z, n_acc, grid, 15, dev)
    b = _run(z, n_acc, grid, 15, dev)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


def test_sts_position_never_reached(dev):
    """Every rollout rejects at the first position: positions 2.. are never
    reached, their AUC is NaN, and every label past position 1 is 0."""
    N, gamma = 2000, 3
    rng = np.random.default_rng(1)
    z = rng.normal(size=(N, gamma)).astype(np.float32)
    n_acc = np.zeros(N, dtype=np.int32)
    grid = W.sts_grid()
    T, e0, e1, auc = _run(z, n_acc, grid, 15, dev)
    ref = OS.sts_fit(z, n_acc, grid, 15, teacher_T=T)
    assert np.isnan(auc[1]) and np.isnan(auc[2]) and np.isnan(auc[0])   # no accepted draft anywhere
    assert np.all(np.abs(e1 - ref["ece_after"]) <= 2.5 / N + 1e-6)


@pytest.mark.parametrize("N", [8192, 8193, 20000])
def test_sts_auc_ties_and_signed_zeros(N, dev):
    """Logits on a coarse grid (most pairs tie) with many exact -0.0 and
    +0.0, at rollout counts on and just past a sort-chunk boundary: the AUC
    is the oracle's pair count exactly (ties count one half, -0 equals +0)."""
    gamma = 5
    rng = np.random.default_rng(N)
    z = (np.round(rng.normal(size=(N, gamma)) * 2) / 4).astype(np.float32)
    zero = rng.random(size=(N, gamma)) < 0.2
    z[zero] = np.where(rng.random(size=int(zero.sum())) < 0.5, np.float32(-0.0), np.float32(0.0))
    n_acc = rng.integers(0, gamma + 1, size=N).astype(np.int32)
    say(f"[sts ties] N={N} gamma={gamma}")
    _, _, _, auc = _run(z, n_acc, W.sts_grid(), 15, dev)
    for k in range(gamma):
        reach = n_acc >= k
        ref = OS.auc_pairs(z[reach, k], (n_acc >= k + 1)[reach])
        assert abs(auc[k] - ref) <= 1e-12, (k, auc[k], ref)
