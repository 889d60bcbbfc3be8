"""GPU greedy verification (bit-exact) and analytic acceptance (within
ACC_TOL of the float64 oracle) through the C ABI: small rounds spanning
several tiles and ragged tails, bf16 and fp32 storage, packed target rows,
argmax ties, and full-size workloads on sampled requests.

ACC_TOL: the kernel's target normaliser is an fp32 log-sum-exp (a few
2^-24 relative on |lse| ~ 12, so p_t within ~1e-6 relative), its
exponentials are fp32, and the sum of up to 1.5e5 terms is accumulated in
fp32, sixteen per lane per tile, then per lane over tiles and across
partials (a few 1e-7 at these sizes); c* <= 1, so 1e-5 absolute leaves an
order of magnitude over the largest error seen (6e-7).  The drafter's
normaliser is the sampler's own output, fed to both sides."""

import sys

import numpy as np
import pytest

from oracle.common import as_f64
from oracle import verify as OV
from semi_ar_draft_round_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ACC_TOL = 1e-5


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from semi_ar_draft_round_amd import binding
    binding.load_library()
    return torch.device("cuda:0")


def _greedy_drafts(tgt64, rng, with_ties_rows=None):
    """Drafts that follow the target's argmax for a random number of positions."""
    R, gp1, V = tgt64.shape
    gamma = gp1 - 1
    am = tgt64.argmax(axis=2)
    x = rng.integers(0, V, size=(R, gamma))
    for q in range(R):
        keep = int(rng.integers(0, gamma + 1))
        x[q, :keep] = am[q, :keep]
    return x.astype(np.int32)


def _store(a, dt, dev):
    from semi_ar_draft_round_amd import device_round as DR
    return DR._dev_store(a, dt, dev)


GREEDY = [
    W.custom("greedy_r20_g5_v1000_bf16", R=20, gamma=5, V=1000, r=32, d=64, seed=21),
    W.custom("greedy_r3_g3_v203_bf16", R=3, gamma=3, V=203, r=32, d=64, seed=22),
    W.custom("greedy_r70_g6_v4100_bf16", R=70, gamma=6, V=4100, r=32, d=64, seed=23),
    W.custom("greedy_r9_g7_v333_f32", R=9, gamma=7, V=333, r=20, d=36, dtype="f32", seed=24),
    W.custom("greedy_r6_g64_v1000_bf16", R=6, gamma=64, V=1000, r=32, d=64, seed=25),
    W.BY_NAME["heavy_r128_g16_v129280"],
]


@pytest.mark.parametrize("w", GREEDY, ids=[w.name for w in GREEDY])
def test_greedy_bit_exact(w, dev):
    from semi_ar_draft_round_amd import binding as B
    say(f"[greedy] {w.name}")
    inp = W.make_inputs(w)
    rng = np.random.default_rng(w.seed)
    tgt = inp.target.copy()
    if w.dtype == "bf16":
        # ties: copy each row's largest logit to a second, random position
        t64 = as_f64(tgt, w.dtype)
        am = t64.argmax(axis=2)
        R, gp1, _ = tgt.shape
        for q in range(R):
            for i in range(0, gp1, 2):
                tgt[q, i, int(rng.integers(0, w.V))] = tgt[q, i, am[q, i]]
    t64 = as_f64(tgt, w.dtype)
    x = _greedy_drafts(t64, rng)
    ell = rng.integers(0, w.gamma + 1, size=w.R).astype(np.int32)
    n_acc, next_tok = B.dspark_verify_greedy(_store(tgt, w.dtype, dev), torch.tensor(x, device=dev),
                                             torch.tensor(ell, device=dev))
    torch.cuda.synchronize()
    ref = OV.verify_greedy(t64, None, x, ell)
    assert n_acc.cpu().numpy().tolist() == ref["n_acc"].tolist()
    assert next_tok.cpu().numpy().tolist() == ref["next_tok"].tolist()
    say(f"  accepted {int(ref['n_acc'].sum())} of {int(ell.sum())}")


def test_greedy_all_accepted_at_max_gamma(dev):
    """gamma = 64 with every admitted draft equal to its row's argmax: the
    accepted prefix is the whole admitted length, and the next token is the
    argmax of row l_r (row 64, the bonus row, when all 64 are admitted)."""
    from semi_ar_draft_round_amd import binding as B
    w = W.custom("greedy_all_r4_g64_v1000_bf16", R=4, gamma=64, V=1000, r=32, d=64, seed=26)
    say(f"[greedy] {w.name}")
    inp = W.make_inputs(w)
    t64 = as_f64(inp.target, w.dtype)
    x = t64.argmax(axis=2)[:, :w.gamma].astype(np.int32)
    ell = np.array([64, 63, 0, 64], dtype=np.int32)
    n_acc, next_tok = B.dspark_verify_greedy(_store(inp.target, w.dtype, dev), torch.tensor(x, device=dev),
                                             torch.tensor(ell, device=dev))
    torch.cuda.synchronize()
    ref = OV.verify_greedy(t64, None, x, ell)
    assert ref["n_acc"].tolist() == ell.tolist()
    assert n_acc.cpu().numpy().tolist() == ell.tolist()
    assert next_tok.cpu().numpy().tolist() == ref["next_tok"].tolist()


def test_greedy_packed_rows_match_dense(dev):
    from semi_ar_draft_round_amd import binding as B
    w = GREEDY[0]
    inp = W.make_inputs(w)
    rng = np.random.default_rng(3)
    t64 = as_f64(inp.target, w.dtype)
    x = _greedy_drafts(t64, rng)
    ell = rng.integers(0, w.gamma + 1, size=w.R).astype(np.int32)
    # pack rows 0..ell[r] of each request, in reverse request order
    rows, row0 = [], np.zeros(w.R, dtype=np.int32)
    for q in reversed(range(w.R)):
        row0[q] = sum(len(r_) for r_ in rows)
        rows.append(inp.target[q, : ell[q] + 1])
    packed = np.concatenate(rows, axis=0)
    n1, t1 = B.dspark_verify_greedy(_store(packed, w.dtype, dev), torch.tensor(x, device=dev),
                                    torch.tensor(ell, device=dev), row0=torch.tensor(row0, device=dev))
    n2, t2 = B.dspark_verify_greedy(_store(inp.target, w.dtype, dev), torch.tensor(x, device=dev),
                                    torch.tensor(ell, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(n1, n2) and torch.equal(t1, t2)


ACC_SMALL = [
    W.BY_NAME["tiny_r1_g4_v1024_f32"],
    W.custom("acc_r20_g5_v1000_bf16", R=20, gamma=5, V=1000, r=256, d=512, seed=31),
    W.custom("acc_r3_g3_v203_bf16", R=3, gamma=3, V=203, r=32, d=64, seed=32),
    W.custom("acc_r70_g6_v4100_r64_bf16", R=70, gamma=6, V=4100, r=64, d=128, seed=33),
    W.custom("acc_r9_g7_v333_f32", R=9, gamma=7, V=333, r=20, d=36, dtype="f32", seed=34),
    W.custom("acc_r5_g64_v1000_bf16", R=5, gamma=64, V=1000, r=64, d=64, seed=35),
    # the sweep that keeps W2t on chip: an odd number of 32-row blocks (9)
    # over groups of two or three tiles, with 16-byte logit loads
    W.custom("acc_r40_g7_v40000_r256_bf16", R=40, gamma=7, V=40000, r=256, d=64, seed=36),
    # V a multiple of 16, so the sweep keeps four tiles of logits in flight
    # (B rows in LDS): 50 rows in groups of 64 at r = 256, 280 rows in groups
    # of 128 at r = 64 (W2t one step ahead), 24 rows in one group of 32 at
    # r = 128; the W2t tiles two steps ahead are the 280-row r = 256 case above
    W.custom("acc_r10_g5_v4096_r256_bf16", R=10, gamma=5, V=4096, r=256, d=64, seed=37),
    W.custom("acc_r70_g4_v8192_r64_bf16", R=70, gamma=4, V=8192, r=64, d=64, seed=38),
    W.custom("acc_r8_g3_v2048_r128_bf16", R=8, gamma=3, V=2048, r=128, d=64, seed=39),
]


def _acceptance_case(w, dev, idx=None):
    from semi_ar_draft_round_amd import binding as B
    from semi_ar_draft_round_amd import device_round as DR
    inp = W.make_inputs(w)
    d = DR.to_device(inp, dev)
    DR.sample(d)                      # the drafts and the sampler's normalisers
    c_star = B.dspark_acceptance(d.target, d.U, d.W1, d.W2t, d.x0, d.x, d.lse)
    torch.cuda.synchronize()
    x = d.x.cpu().numpy().astype(np.int64)
    lse = d.lse.cpu().numpy().astype(np.float64)
    got = c_star.cpu().numpy().astype(np.float64)
    idx = np.arange(w.R) if idx is None else idx
    ref = OV.analytic_acceptance(as_f64(inp.target[idx], w.dtype), None, as_f64(inp.U[idx], w.dtype),
                                 as_f64(inp.E, w.dtype), as_f64(inp.W2t, w.dtype), inp.x0[idx].astype(np.int64),
                                 x[idx], lse[idx])
    err = np.abs(got[idx] - ref)
    assert err.max() <= ACC_TOL, (err.max(), np.unravel_index(err.argmax(), err.shape))
    assert np.all((got >= 0) & (got <= 1 + ACC_TOL))
    return err.max(), got


@pytest.mark.parametrize("w", ACC_SMALL, ids=[w.name for w in ACC_SMALL])
def test_acceptance_small(w, dev):
    say(f"[acceptance] {w.name}")
    e, _ = _acceptance_case(w, dev)
    say(f"  max |c* - oracle| = {e:.2e}")


@pytest.mark.parametrize("name", ["batch_r32_g16_v151936", "heavy_r128_g16_v129280"])
def test_acceptance_full_size_sampled(name, dev):
    w = W.BY_NAME[name]
    rng = np.random.default_rng(9)
    idx = np.sort(rng.choice(w.R, size=min(w.R, 3), replace=False))
    say(f"[acceptance] {name}: oracle on requests {idx.tolist()}")
    e, _ = _acceptance_case(w, dev, idx)
    say(f"  max |c* - oracle| = {e:.2e}")


def test_acceptance_packed_rows_match_dense(dev):
    from semi_ar_draft_round_amd import binding as B
    from semi_ar_draft_round_amd import device_round as DR
    w = ACC_SMALL[1]
    inp = W.make_inputs(w)
    d = DR.to_device(inp, dev)
    DR.sample(d)
    dense = B.dspark_acceptance(d.target, d.U, d.W1, d.W2t, d.x0, d.x, d.lse).clone()
    rows, row0 = [], np.zeros(w.R, dtype=np.int32)
    for q in reversed(range(w.R)):
        row0[q] = sum(len(r_) for r_ in rows)
        rows.append(inp.target[q, : w.gamma])          # rows 0 .. gamma-1 are what it reads
    packed = _store(np.concatenate(rows, axis=0), w.dtype, dev)
    got = B.dspark_acceptance(packed, d.U, d.W1, d.W2t, d.x0, d.x, d.lse, row0=torch.tensor(row0, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(got, dense)
