"""GPU scheduler on the pages' worked examples and adversarial tie patterns
(bit-exact against the oracle), and the two verification invariants measured
on the GPU path with the request axis as the trial axis."""

import json
import os
import sys

import numpy as np
import pytest
from scipy import stats

from oracle.schedule import admit

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from semi_ar_draft_round_amd import binding
    binding.load_library()
    return torch.device("cuda:0")


def gpu_schedule(c, sps, dev):
    from semi_ar_draft_round_amd import binding as B
    ell, A, th = B.dspark_schedule(torch.tensor(np.asarray(c, dtype=np.float32), device=dev),
                                   torch.tensor(np.asarray(sps, dtype=np.float64), device=dev))
    torch.cuda.synchronize()
    return ell.cpu().numpy(), int(A.cpu()[0]), float(th.cpu()[0])


def assert_same(c, sps, dev):
    ref = admit(np.asarray(c, dtype=np.float32), np.asarray(sps, dtype=np.float64))
    ell, A, th = gpu_schedule(c, sps, dev)
    assert ell.tolist() == ref["ell"].tolist()
    assert A == ref["A"]
    assert th == ref["theta_best"]
    return ref


@pytest.mark.parametrize("name", ["scheduler_single_request.json", "scheduler_two_requests.json",
                                  "scheduler_three_requests.json"])
def test_worked_examples_on_gpu(name, dev):
    say(f"[schedule] {name}")
    g = json.load(open(os.path.join(GOLD, name)))
    c = np.array(g["c"], dtype=np.float32)
    if c.ndim == 1:
        c = c[None, :]
    ref = assert_same(c, np.array(g["sps"], dtype=np.float64), dev)
    want = g.get("ell", [g.get("admit")])
    assert ref["ell"].tolist() == want


def test_appendix_a_eq9_on_gpu(dev):
    say("[schedule] appendix A eq 9")
    g = json.load(open(os.path.join(GOLD, "appendix_a.json")))["eq9"]
    for c2 in (0.9, 0.0):
        ref = assert_same(np.array([[g["a1"], c2]]), np.array(g["sps"]), dev)
        assert ref["ell"].tolist() == [0]


def random_case(rng, R, gamma, ties):
    c = rng.uniform(0.05, 1.0, size=(R, gamma)).astype(np.float32)
    if ties:
        c[rng.uniform(size=c.shape) < 0.3] = 1.0
        c[rng.uniform(size=c.shape) < 0.1] = 0.0
        c[: R // 2] = c[R // 2: 2 * (R // 2)]         # identical requests: ties across r
    n = R * (1 + gamma)
    kind = rng.integers(0, 3)
    B = np.arange(1, n + 1, dtype=np.float64)
    if kind == 0:
        sps = np.floor(4096000.0 / (B + 2048.0))
    elif kind == 1:
        sps = 8.0 * np.floor(1000.0 / (1.0 + np.maximum(0, B - R) / 64.0) / 8.0)
    else:
        sps = np.sort(rng.integers(1, 5, size=n).astype(np.float64) * 250.0)[::-1].copy()
    return c, sps


@pytest.mark.parametrize("seed", range(10))
def test_random_batches_bit_exact(seed, dev):
    rng = np.random.default_rng(500 + seed)
    R = int(rng.integers(1, 200))
    gamma = int(rng.integers(1, 17))
    say(f"[schedule] random seed={seed} R={R} gamma={gamma}")
    c, sps = random_case(rng, R, gamma, ties=bool(seed % 2))
    assert_same(c, sps, dev)


def test_largest_batch_bit_exact(dev):
    """R (1 + gamma) = 8177: 7696 slots, the full 8192-key sort."""
    rng = np.random.default_rng(77)
    R, gamma = 481, 16
    say(f"[schedule] R={R} gamma={gamma}")
    c = rng.uniform(0.3, 1.0, size=(R, gamma)).astype(np.float32)
    B = np.arange(1, R * (1 + gamma) + 1, dtype=np.float64)
    assert_same(c, np.floor(1e7 / (B + 100.0)), dev)
    assert_same(c, np.full(R * (1 + gamma), 3.0), dev)   # flat: admit every slot


def test_equal_theta_stops_on_gpu(dev):
    say("[schedule] equal theta")
    ell, A, th = gpu_schedule(np.array([[0.5]]), np.array([3.0, 2.0]), dev)
    assert ell.tolist() == [0] and A == 0 and th == 3.0


def _invariant_instance(V, seed):
    rng = np.random.default_rng(seed)
    lp_d = rng.normal(0, 1.0, size=V)
    lp_t = rng.normal(0, 1.0, size=V)
    return lp_d, lp_t


def test_gpu_lossless_and_acceptance_rate(dev):
    """Invariants (a) and (b) on the GPU path: R = 60000 copies of one request
    with V = 8, one drafted position, every draft admitted (ell = 1)."""
    from semi_ar_draft_round_amd import binding as B
    from semi_ar_draft_round_amd import workloads as W
    say("[stats] lossless / acceptance rate, R=60000, V=8")
    R, gamma, V, r = 60000, 1, 8, 32
    lp_d, lp_t = _invariant_instance(V, 3)
    # bf16-representable logits so both sides see exactly these values
    lp_d = W.bf16_to_f32(W.bf16_bits(lp_d.astype(np.float32))).astype(np.float64)
    lp_t = W.bf16_to_f32(W.bf16_bits(lp_t.astype(np.float32))).astype(np.float64)
    p_d = np.exp(lp_d - lp_d.max()); p_d /= p_d.sum()
    p_t = np.exp(lp_t - lp_t.max()); p_t /= p_t.sum()
    bf = lambda a: torch.from_numpy(W.bf16_bits(np.ascontiguousarray(a, dtype=np.float32)).view(np.int16)).view(torch.bfloat16).to(dev)
    U = bf(np.broadcast_to(lp_d, (R, gamma, V)))
    tgt = bf(np.broadcast_to(np.stack([lp_t, lp_t]), (R, gamma + 1, V)))
    W1 = bf(np.zeros((V, r)))
    W2t = bf(np.zeros((V, r)))
    rng = np.random.default_rng(11)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    G = f32(W.gumbel_from_uniform(W.odd_uniform(rng, (gamma, 1, R))))
    g = f32(W.gumbel_from_uniform(W.odd_uniform(rng, (R, gamma, W.CHUNK))))
    x0 = torch.zeros(R, dtype=torch.int32, device=dev)
    x, lse, logit = B.dspark_markov_sample(U, W1, W2t, x0, G, g)
    ell = torch.ones(R, dtype=torch.int32, device=dev)
    u_acc = f32(W.odd_uniform(rng, (R, gamma)))
    u_res = f32(W.odd_uniform(rng, (R,)))
    n_acc, nxt = B.dspark_verify(tgt, U, W1, W2t, x0, x, lse, logit, ell, u_acc, u_res)
    torch.cuda.synchronize()
    xh = x.cpu().numpy()[:, 0]
    n = n_acc.cpu().numpy()
    t = nxt.cpu().numpy()
    # the drafts follow p_d
    assert stats.chisquare(np.bincount(xh, minlength=V), R * p_d).pvalue > 1e-4
    first = np.where(n == 1, xh, t)
    p = stats.chisquare(np.bincount(first, minlength=V), R * p_t).pvalue
    acc = n.mean()
    want = 1.0 - 0.5 * np.abs(p_d - p_t).sum()
    z = (acc - want) / np.sqrt(want * (1 - want) / R)
    say(f"  chi2 p={p:.3g}, accept {acc:.4f} vs {want:.4f} (z={z:.2f})")
    assert p > 1e-4
    assert abs(z) < 4.5


@pytest.mark.parametrize("R,gamma", [(4095, 1), (126, 64), (1, 64), (2, 1), (100, 3), (33, 31)])
def test_extreme_shapes_bit_exact(R, gamma, dev):
    """Runs of one key (gamma = 1, 4095 requests), of the largest length
    (gamma = 64), and shapes whose slot counts are not multiples of the
    ranking's 32-key work groups: bit-exact with and without ties."""
    for ties in (False, True):
        rng = np.random.default_rng(R * 1000 + gamma + (7 if ties else 0))
        say(f"[schedule] R={R} gamma={gamma} ties={ties}")
        c, sps = random_case(rng, R, gamma, ties=ties)
        assert_same(c, sps, dev)
