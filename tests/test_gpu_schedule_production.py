"""GPU production scheduler (dspark_schedule_ex): the whole-walk capacity
and the capacity fill, bit-exact against the oracle on the pages' table,
hand-worked stepped tables, random and tie-heavy batches, the largest batch,
the two-round production chain with the capacity passed device to device,
and HIP-graph replays."""

import json
import os
import sys

import numpy as np
import pytest

from oracle.schedule import admit_capacity, admit_full_scan, production_schedule

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


def run(c, sps, mode, K, dev):
    from semi_ar_draft_round_amd import binding as B
    cap = None if K is None else torch.tensor([K], dtype=torch.int32, device=dev)
    ell, A, th = B.dspark_schedule_ex(torch.tensor(np.asarray(c, dtype=np.float32), device=dev),
                                      torch.tensor(np.asarray(sps, dtype=np.float64), device=dev), mode, cap)
    torch.cuda.synchronize()
    return ell.cpu().numpy(), int(A.cpu()[0]), float(th.cpu()[0])


def same_whole_walk(c, sps, dev):
    from semi_ar_draft_round_amd import binding as B
    ref = admit_full_scan(np.asarray(c, dtype=np.float32), np.asarray(sps, dtype=np.float64))
    ell, A, th = run(c, sps, B.SCHED_WHOLE_WALK, None, dev)
    assert ell.tolist() == ref["ell"].tolist()
    assert A == ref["A"]
    assert th == ref["theta_best"]
    return ref


def same_capacity(c, sps, K, dev):
    from semi_ar_draft_round_amd import binding as B
    ref = admit_capacity(np.asarray(c, dtype=np.float32), np.asarray(sps, dtype=np.float64), K)
    ell, A, th = run(c, sps, B.SCHED_CAPACITY, K, dev)
    assert ell.tolist() == ref["ell"].tolist(), K
    assert A == ref["A"], K
    assert th == ref["theta_best"], K
    return ref


def test_pages_table_and_hand_examples(dev):
    say("[production] worked examples")
    g = json.load(open(os.path.join(GOLD, "scheduler_two_requests.json")))
    ref = same_whole_walk(np.array(g["c"]), np.array(g["sps"]), dev)
    assert ref["A"] == 1
    ones = np.ones((1, 3))
    assert same_whole_walk(ones, [100.0, 60.0, 40.0, 40.0], dev)["A"] == 3    # past a local peak
    assert same_whole_walk(ones, [100.0, 60.0, 40.0, 30.0], dev)["A"] == 1    # smallest m on ties
    for K in (-5, 0, 1, 2, 3, 99):
        same_capacity(ones, [100.0, 60.0, 40.0, 40.0], K, dev)


def stepped_case(rng, R, gamma, ties):
    c = rng.uniform(0.05, 1.0, size=(R, gamma)).astype(np.float32)
    if ties:
        c[rng.uniform(size=c.shape) < 0.3] = 1.0
        c[rng.uniform(size=c.shape) < 0.1] = 0.0
        c[: R // 2] = c[R // 2: 2 * (R // 2)]
    n = R * (1 + gamma)
    B = np.arange(1, n + 1, dtype=np.float64)
    kind = rng.integers(0, 3)
    if kind == 0:        # staircase of the latency and batch workloads
        sps = 8.0 * np.floor(1000.0 / (1.0 + np.maximum(0, B - 64) / 256.0) / 8.0)
    elif kind == 1:      # sharp cliffs with plateaus
        drops = np.where(rng.random(n) < 0.05, rng.uniform(0.1, 0.4, size=n), 0.0)
        drops[0] = 0.0
        sps = np.floor(2000.0 * np.cumprod(1.0 - drops))
    else:                # smooth
        sps = np.floor(4096000.0 / (B + 2048.0))
    return c, sps


@pytest.mark.parametrize("seed", range(12))
def test_random_batches_bit_exact(seed, dev):
    rng = np.random.default_rng(900 + seed)
    R = int(rng.integers(1, 200))
    gamma = int(rng.integers(1, 17))
    say(f"[production] random seed={seed} R={R} gamma={gamma}")
    c, sps = stepped_case(rng, R, gamma, ties=bool(seed % 2))
    ref = same_whole_walk(c, sps, dev)
    for K in (0, 1, ref["A"], R * gamma // 2, R * gamma, R * gamma + 7, -1):
        same_capacity(c, sps, K, dev)


@pytest.mark.parametrize("R,gamma", [(481, 16), (126, 64)])
def test_largest_batch_bit_exact(R, gamma, dev):
    """The largest batches the slot limit admits: R (1 + gamma) = 8177 and 8190."""
    rng = np.random.default_rng(78 + gamma)
    say(f"[production] R={R} gamma={gamma}")
    c = rng.uniform(0.3, 1.0, size=(R, gamma)).astype(np.float32)
    B = np.arange(1, R * (1 + gamma) + 1, dtype=np.float64)
    sps = 8.0 * np.floor(1e5 / (1.0 + np.maximum(0, B - 512) / 512.0) / 8.0)
    same_whole_walk(c, sps, dev)
    same_whole_walk(c, np.full(R * (1 + gamma), 3.0), dev)   # flat: every slot
    for K in (0, 4000, R * gamma):
        same_capacity(c, sps, K, dev)


def test_production_chain_device_to_device(dev):
    """Six rounds: round t fills the capacity that the whole-walk call made on
    round t - 2, read from that call's `admitted` output on the device."""
    from semi_ar_draft_round_amd import binding as B
    rng = np.random.default_rng(5)
    R, gamma = 64, 8
    n = R * (1 + gamma)
    Bs = np.arange(1, n + 1, dtype=np.float64)
    sps = 8.0 * np.floor(1000.0 / (1.0 + np.maximum(0, Bs - 64) / 128.0) / 8.0)
    rounds = [rng.uniform(0.2, 1.0, size=(R, gamma)).astype(np.float32) for _ in range(6)]
    ref = production_schedule(rounds, sps, K_init=40)
    sps_d = torch.tensor(sps, device=dev)
    caps = [torch.tensor([40], dtype=torch.int32, device=dev) for _ in range(2)]
    for t, c in enumerate(rounds):
        say(f"[production] chain round {t}")
        c_d = torch.tensor(c, device=dev)
        ell, A, th = B.dspark_schedule_ex(c_d, sps_d, B.SCHED_CAPACITY, caps[t])
        _, K_next, _ = B.dspark_schedule_ex(c_d, sps_d, B.SCHED_WHOLE_WALK)
        caps.append(K_next)
        torch.cuda.synchronize()
        assert ell.cpu().tolist() == ref[t]["ell"].tolist()
        assert int(A.cpu()[0]) == ref[t]["A"]
        assert float(th.cpu()[0]) == ref[t]["theta_best"]


def test_graph_replays_match_eager(dev):
    from semi_ar_draft_round_amd import binding as B
    rng = np.random.default_rng(17)
    R, gamma = 128, 16
    c, sps = stepped_case(rng, R, gamma, ties=True)
    c_d = torch.tensor(c, device=dev)
    sps_d = torch.tensor(sps, device=dev)
    cap = torch.tensor([700], dtype=torch.int32, device=dev)
    outs = [torch.empty(R, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
            torch.empty(1, dtype=torch.float64, device=dev)]
    outs2 = [torch.empty(R, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
             torch.empty(1, dtype=torch.float64, device=dev)]
    eager_cap = [t.clone() for t in B.dspark_schedule_ex(c_d, sps_d, B.SCHED_CAPACITY, cap)]
    eager_ww = [t.clone() for t in B.dspark_schedule_ex(c_d, sps_d, B.SCHED_WHOLE_WALK)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            B.dspark_schedule_ex(c_d, sps_d, B.SCHED_CAPACITY, cap, *outs)
            B.dspark_schedule_ex(c_d, sps_d, B.SCHED_WHOLE_WALK, None, *outs2)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        say(f"[production] graph replay {rep}")
        for t in outs + outs2:
            t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs + outs2, eager_cap + eager_ww):
            assert torch.equal(a, b)
