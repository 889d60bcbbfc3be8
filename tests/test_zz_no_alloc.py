"""The allocation-free scheduler, dspark_schedule_noalloc, against
dspark_schedule_ex with a caller workspace: bit-exact ell, A and Theta_best
under all three admission rules, on two calls in a row on one device (the
second with a smaller batch, which reuses the first call's stale scratch)."""

import sys

import numpy as np
import pytest

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


def _batch(R, gamma, seed, dev):
    """Confidences with ties and saturated entries, and a stepped table."""
    rng = np.random.default_rng(seed)
    c = rng.uniform(0.3, 1.0, size=(R, gamma)).astype(np.float32)
    c[rng.random((R, gamma)) < 0.2] = 1.0
    c[rng.random((R, gamma)) < 0.1] = 0.5
    w = W.custom("noalloc", R=R, gamma=gamma, V=64, r=32, d=16, seed=seed)
    sps = W.make_sps(w)
    return (torch.from_numpy(c).to(dev), torch.from_numpy(np.ascontiguousarray(sps)).to(dev))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_noalloc_matches_workspace_call(mode, dev):
    from semi_ar_draft_round_amd import binding as B
    for R, gamma, seed in ((481, 16, 3), (37, 5, 4)):          # the largest batch first, then a smaller one
        say(f"[noalloc] mode {mode} R {R} gamma {gamma}")
        c, sps = _batch(R, gamma, seed, dev)
        cap = torch.tensor([R * gamma // 3], dtype=torch.int32, device=dev) if mode == 2 else None
        ws = torch.full((B.dspark_workspace_size(B.WS_SCHEDULE, R, gamma, 0, 0),), 0xFF, dtype=torch.uint8,
                        device=dev)
        e1, a1, t1 = B.dspark_schedule_ex(c, sps, mode, cap, ws=ws)
        e2, a2, t2 = B.dspark_schedule_noalloc(c, sps, mode, cap)
        torch.cuda.synchronize()
        assert e1.cpu().tolist() == e2.cpu().tolist()
        assert int(a1.cpu()[0]) == int(a2.cpu()[0])
        assert float(t1.cpu()[0]) == float(t2.cpu()[0])


def test_noalloc_rejects_batches_beyond_its_scratch(dev):
    from semi_ar_draft_round_amd import binding as B
    c, sps = _batch(482, 16, 5, dev)                           # 482 * 17 > 8191
    with pytest.raises(B.DSparkError):
        B.dspark_schedule_noalloc(c, sps, 0)
