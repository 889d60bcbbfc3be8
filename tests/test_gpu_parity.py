"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Small workloads are checked on every output; the large ones (the sizes the
benchmark times, in the same launch configuration) on a sample of requests
the oracle recomputes one by one, plus the whole-batch scheduler."""

import sys

import numpy as np
import pytest

from semi_ar_draft_round_amd import workloads as W

from parity import check_confidence, check_sample, check_schedule, check_verify

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


def run_gpu(inp, dev):
    from semi_ar_draft_round_amd import device_round as DR
    d = DR.to_device(inp, dev)
    DR.run_round(d)
    return d, DR.outputs_to_host(d)


SMALL = [
    W.BY_NAME["tiny_r1_g4_v1024_f32"],
    W.custom("ragged_r20_g5_v1000_bf16", R=20, gamma=5, V=1000, r=256, d=512, seed=11),
    W.custom("odd_v_r3_g3_v203_bf16", R=3, gamma=3, V=203, r=32, d=64, seed=12),
    W.custom("r130_g4_v700_r128_bf16", R=130, gamma=4, V=700, r=128, d=256, seed=13, temperatures=True),
    W.custom("r70_g6_v4100_r64_bf16", R=70, gamma=6, V=4100, r=64, d=128, seed=14),
    W.custom("f32_r9_g7_v333", R=9, gamma=7, V=333, r=20, d=36, dtype="f32", seed=15),
    W.custom("gmax_r5_g64_v1000_bf16", R=5, gamma=64, V=1000, r=64, d=64, seed=16),
    # 18752 chunk masses per request: more than the residual draw keeps in
    # registers, so it scans them from memory
    W.custom("bigv_r3_g2_v300000_bf16", R=3, gamma=2, V=300000, r=32, d=64, seed=62),
    # the instantiations the benchmark runs, on every request: 128-request
    # groups with r = 256 (sampler and residual sweep at 4 request quarters and
    # 16 k-steps), with V a multiple of 16 (16-byte logit loads) and not
    # (token-by-token loads), and two request groups side by side
    W.custom("wide_r130_g4_v4096_r256_bf16", R=130, gamma=4, V=4096, r=256, d=128, seed=18),
    W.custom("wide_r130_g4_v4100_r256_bf16", R=130, gamma=4, V=4100, r=256, d=128, seed=19),
    W.custom("wide_r256_g3_v2048_r256_bf16", R=256, gamma=3, V=2048, r=256, d=64, seed=20, temperatures=True),
    # the per-block-barrier kernel with the fewest blocks it takes (3), with
    # every compute unit holding two or three tiles; and a ragged last block
    # of 8 at 7 blocks
    W.custom("pipe_r96_g5_v40000_r256_bf16", R=96, gamma=5, V=40000, r=256, d=64, seed=23),
    W.custom("pipe_r200_g3_v20000_r256_bf16", R=200, gamma=3, V=20000, r=256, d=64, seed=24),
    # the per-block kernel at r = 32 (every k-step in registers), and at its
    # largest batch, 32 blocks
    W.custom("pipe_r100_g5_v3000_r32_bf16", R=100, gamma=5, V=3000, r=32, d=64, seed=28),
    W.custom("pipe_r1024_g2_v640_r64_bf16", R=1024, gamma=2, V=640, r=64, d=64, seed=29),
    # single request blocks with more than eight tiles per compute unit (the
    # resident kernel's LDS-held ninth and tenth tiles): some groups with a
    # ninth tile, every group with ten (the largest vocabulary it takes),
    # and a full block with V not a multiple of 16
    W.custom("res9_r3_g3_v140000_r256_bf16", R=3, gamma=3, V=140000, r=256, d=64, seed=25),
    W.custom("res10_r2_g4_v163840_r256_bf16", R=2, gamma=4, V=163840, r=256, d=64, seed=26),
    W.custom("res10_r32_g2_v150003_r256_bf16", R=32, gamma=2, V=150003, r=256, d=64, seed=27),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_round_full_parity(w, dev):
    say(f"[parity] {w.name}")
    inp = W.make_inputs(w)
    if w.name.startswith("odd_v"):
        inp.x0[1] = -1                                  # no previous token: B_1 = 0
    _, out = run_gpu(inp, dev)
    idx = np.arange(w.R)
    rs = check_sample(inp, out, idx)
    rc = check_confidence(inp, out, idx)
    rsch = check_schedule(inp.sps, out)
    rv = check_verify(inp, out, idx)
    say(f"  sample {rs}\n  conf {rc}\n  sched {rsch}\n  verify {rv}")


LARGE = [W.BY_NAME[n] for n in ("latency_r1_g16_v151936", "batch_r32_g16_v151936",
                                 "heavy_r128_g16_v129280", "full_r256_g16_v129280_sts")]


@pytest.mark.parametrize("w", LARGE, ids=[w.name for w in LARGE])
def test_full_size_sampled_parity(w, dev):
    say(f"[parity] {w.name}: drawing inputs")
    inp = W.make_inputs(w)
    say(f"[parity] {w.name}: GPU round")
    _, out = run_gpu(inp, dev)
    rng = np.random.default_rng(7)
    n = min(w.R, 6)
    idx = np.sort(rng.choice(w.R, size=n, replace=False))
    # always include the requests with the longest admitted prefix
    longest = np.argsort(-out["ell"], kind="stable")[:2]
    idx = np.unique(np.concatenate([idx, longest]))
    say(f"[parity] {w.name}: oracle on requests {idx.tolist()}, A = {out['A']}")
    rs = check_sample(inp, out, idx)
    rc = check_confidence(inp, out, idx)
    rsch = check_schedule(inp.sps, out)
    rv = check_verify(inp, out, idx)
    say(f"  sample {rs}\n  conf {rc}\n  sched {rsch}\n  verify {rv}")
    assert np.all((out["x"] >= 0) & (out["x"] < w.V))
    assert np.all((out["c"] >= 0) & (out["c"] <= 1))
    assert np.all(out["n_acc"] <= out["ell"])
    assert np.all((out["next_tok"] >= 0) & (out["next_tok"] < w.V))


MANY = [W.custom(f"many_r33000_g2_v{V}_bf16", R=33000, gamma=2, V=V, r=32, d=64, seed=51) for V in (320, 203)]


@pytest.mark.parametrize("w", MANY, ids=[w.name for w in MANY])
def test_many_requests_sampled_parity(w, dev):
    """More request groups of 128 than compute units: the sampler takes one
    launch per position instead of the persistent grid, and the target
    normalisers walk every (row, part) item instead of a prefix of the
    needed rows.  V = 320 takes the 16-byte vector loads, V = 203 the scalar
    ones.  The scheduler's slot limit is far below R (1 + gamma), so the
    admitted lengths are drawn (seeded) and sample and verify are called
    directly; requested rows include the ragged last group."""
    from semi_ar_draft_round_amd import device_round as DR
    say(f"[parity] {w.name}: drawing inputs")
    inp = W.make_inputs(w)
    d = DR.to_device(inp, dev)
    ell = np.random.default_rng(5).integers(0, w.gamma + 1, size=w.R).astype(np.int32)
    d.ell.copy_(torch.from_numpy(ell))
    say(f"[parity] {w.name}: GPU sample + verify")
    DR.sample(d)
    DR.verify(d)
    torch.cuda.synchronize()
    out = dict(x=d.x.cpu().numpy(), lse=d.lse.cpu().numpy(), logit=d.logit.cpu().numpy(), ell=ell,
               n_acc=d.n_acc.cpu().numpy(), next_tok=d.next_tok.cpu().numpy())
    rng = np.random.default_rng(9)
    idx = np.unique(np.concatenate([rng.choice(w.R, size=6, replace=False), [0, 32767, 32768, w.R - 1]]))
    say(f"[parity] {w.name}: oracle on requests {idx.tolist()}")
    rs = check_sample(inp, out, idx)
    rv = check_verify(inp, out, idx)
    say(f"  sample {rs}\n  verify {rv}")
    assert np.all((out["x"] >= 0) & (out["x"] < w.V))
    assert np.all(np.isfinite(out["lse"])) and np.all(np.isfinite(out["logit"]))
    assert np.all((out["n_acc"] >= 0) & (out["n_acc"] <= ell))
    assert np.all((out["next_tok"] >= 0) & (out["next_tok"] < w.V))


@pytest.mark.parametrize("R", [20, 100])
def test_very_negative_logits_with_a_phantom_tile(R, dev):
    """Logits near -200 (U shifted by -200) and an odd tile count (V = 700:
    11 tiles of 64, so one work group also sweeps a phantom tile past V whose
    chunks hold no logit).  Folding an empty chunk must not lift the running
    maximum: with every real logit below about -87 that would flush the
    work group's partial sum to zero and corrupt lse."""
    w = W.custom(f"neg200_r{R}_g3_v700_r256_bf16", R=R, gamma=3, V=700, r=256, d=64, seed=22)
    say(f"[parity] {w.name}")
    inp = W.make_inputs(w)
    inp.U = W.bf16_bits(W.bf16_to_f32(inp.U) - np.float32(200.0))
    _, out = run_gpu(inp, dev)
    idx = np.arange(w.R)
    rs = check_sample(inp, out, idx)
    rv = check_verify(inp, out, idx)
    say(f"  sample {rs}\n  verify {rv}")
    assert np.all(out["lse"] < -150.0)


def test_free_running_round_equals_oracle_round(dev):
    """The whole round on the GPU, free running (no teacher forcing), equals
    the oracle's run_round token for token on the tiny fp32 workload: the
    drafted tokens, the admitted lengths, A, the accepted lengths and the
    next tokens; lse, logit, c and Theta_best within the parity tolerances."""
    from oracle.round import run_round as oracle_round
    w = W.BY_NAME["tiny_r1_g4_v1024_f32"]
    say(f"[parity] free-running round {w.name}")
    for rnd in range(3):
        inp = W.make_inputs(w, round_index=rnd)
        _, out = run_gpu(inp, dev)
        ref = oracle_round(inp)
        assert out["x"].tolist() == ref["x"].tolist(), rnd
        assert out["ell"].tolist() == ref["ell"].tolist(), rnd
        assert out["A"] == ref["A"], rnd
        # Theta_best is bit-exact given the same confidences (checked next);
        # the oracle's free-running c comes from its own float64 dot products,
        # which round to fp32 differently from the GPU's in the last place
        check_schedule(inp.sps, out)
        assert out["theta_best"] == pytest.approx(ref["theta_best"], rel=1e-6), rnd
        assert out["n_acc"].tolist() == ref["n_acc"].tolist(), rnd
        assert out["next_tok"].tolist() == ref["next_tok"].tolist(), rnd
        np.testing.assert_allclose(out["lse"], ref["lse"], rtol=1e-5)
        np.testing.assert_allclose(out["logit"], ref["logit"], rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(out["c"], ref["c"], rtol=1e-5)


@pytest.mark.parametrize("R", [24, 100, 200])
def test_cancelled_sampler_reports_time_out(R, dev):
    """dspark_markov_sample_ex with its cancel word set: the persistent
    launch's grid-barrier waits give up at once (every work group exits
    normally), the status word reads DSPARK_ETIMEOUT and every token is the
    -1 sentinel with NaN lse and logit.  With the word cleared, the same call
    matches dspark_markov_sample followed by dspark_confidence bit for bit."""
    from semi_ar_draft_round_amd import binding as B
    from semi_ar_draft_round_amd import device_round as DR
    w = W.custom(f"cancel_r{R}_g4_v1500", R=R, gamma=4, V=1500, r=256, d=128, seed=43, temperatures=True)
    inp = W.make_inputs(w)
    say(f"[parity] {w.name}")
    d = DR.to_device(inp, dev)
    cancel = torch.ones(1, dtype=torch.int32, device=dev)
    status = torch.full((1,), -9, dtype=torch.int32, device=dev)
    x, lse, logit, c, z, st = B.dspark_markov_sample_ex(d.U, d.W1, d.W2t, d.x0, d.G, d.g, h=d.h, w=d.w, T=d.T,
                                                        z=torch.empty_like(d.z), cancel=cancel, status=status)
    torch.cuda.synchronize()
    assert int(st.cpu()[0]) == 6
    assert np.all(x.cpu().numpy() == -1)
    assert np.all(np.isnan(lse.cpu().numpy())) and np.all(np.isnan(logit.cpu().numpy()))
    cancel.zero_()
    x, lse, logit, c, z, st = B.dspark_markov_sample_ex(d.U, d.W1, d.W2t, d.x0, d.G, d.g, h=d.h, w=d.w, T=d.T,
                                                        z=torch.empty_like(d.z), cancel=cancel, status=status)
    DR.sample(d)
    DR.confidence(d)
    torch.cuda.synchronize()
    assert int(st.cpu()[0]) == 0
    for a, b in ((x, d.x), (lse, d.lse), (logit, d.logit), (c, d.c), (z, d.z)):
        np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())


def test_all_accepted_at_max_gamma(dev):
    """gamma = 64 with every draft admitted and accepted, so the bonus row 64
    is normalised in the accept kernel's second pass over the rows and the
    next token is the bonus draw from it.  W1 = 0 makes p_d = softmax(U_k);
    the target row k is U_k with the drafted token's logit raised by 2, so
    p_t(x_k) > p_d(x_k) and every accept test passes by a wide margin.  One
    request is admitted 63 drafts (its bonus is row 63) and one none."""
    from semi_ar_draft_round_amd import device_round as DR
    w = W.custom("accept_all_r4_g64_v1000_bf16", R=4, gamma=64, V=1000, r=64, d=64, seed=17)
    say(f"[parity] {w.name}")
    inp = W.make_inputs(w)
    inp.E[:] = 0
    d = DR.to_device(inp, dev)
    DR.sample(d)
    torch.cuda.synchronize()
    x = d.x.cpu().numpy()
    u = W.bf16_to_f32(inp.U)
    t = np.concatenate([u, u[:, -1:, :]], axis=1)            # row gamma: a copy of row gamma - 1
    rows = np.arange(w.R)[:, None]
    t[rows, np.arange(w.gamma)[None, :], x] += 2.0
    inp.target = W.bf16_bits(t.astype(np.float32))
    d.target.copy_(DR.to_device(inp, dev).target)
    ell = np.array([64, 63, 0, 64], dtype=np.int32)
    d.ell.copy_(torch.from_numpy(ell))
    DR.verify(d)
    torch.cuda.synchronize()
    out = dict(x=x, lse=d.lse.cpu().numpy(), logit=d.logit.cpu().numpy(), ell=ell,
               n_acc=d.n_acc.cpu().numpy(), next_tok=d.next_tok.cpu().numpy())
    idx = np.arange(w.R)
    rs = check_sample(inp, out, idx)
    rv = check_verify(inp, out, idx)
    say(f"  sample {rs}\n  verify {rv}")
    assert out["n_acc"].tolist() == ell.tolist()


def test_packed_target_rows_match_dense(dev):
    """A flattened ragged verify batch (row0 offsets) gives the dense result."""
    from semi_ar_draft_round_amd import binding as B
    from semi_ar_draft_round_amd import device_round as DR
    w = W.custom("packed_r12_g5_v900", R=12, gamma=5, V=900, r=64, d=64, seed=21)
    inp = W.make_inputs(w)
    say(f"[parity] {w.name}")
    d, out = run_gpu(inp, dev)
    ell = out["ell"]
    rows, row0 = [], []
    for r in range(w.R):
        row0.append(len(rows))
        rows.extend(range(r * (w.gamma + 1), r * (w.gamma + 1) + ell[r] + 1))
    packed = d.target.reshape(w.R * (w.gamma + 1), w.V)[torch.tensor(rows, device=dev)].contiguous()
    row0_t = torch.tensor(row0, dtype=torch.int32, device=dev)
    n2, t2 = B.dspark_verify(packed, d.U, d.W1, d.W2t, d.x0, d.x, d.lse, d.logit, d.ell,
                             d.u_acc, d.u_res, row0=row0_t)
    torch.cuda.synchronize()
    assert n2.cpu().numpy().tolist() == out["n_acc"].tolist()
    assert t2.cpu().numpy().tolist() == out["next_tok"].tolist()


def test_determinism_and_workspace_poison(dev):
    from semi_ar_draft_round_amd import device_round as DR
    w = W.custom("det_r40_g6_v2000", R=40, gamma=6, V=2000, r=256, d=256, seed=31)
    inp = W.make_inputs(w)
    say(f"[parity] {w.name}")
    d = DR.to_device(inp, dev)
    DR.run_round(d)
    a = DR.outputs_to_host(d)
    d.ws_sample.fill_(0xFF)                       # NaN bit patterns everywhere
    d.ws_verify.fill_(0xFF)
    DR.run_round(d)
    b = DR.outputs_to_host(d)
    for k in a:
        np.testing.assert_array_equal(np.asarray(a[k]), np.asarray(b[k]), err_msg=k)


def test_graph_capture_replays_match_eager(dev):
    from semi_ar_draft_round_amd import device_round as DR
    w = W.custom("graph_r24_g4_v1500", R=24, gamma=4, V=1500, r=256, d=128, seed=41)
    inp = W.make_inputs(w)
    say(f"[parity] {w.name}")
    d = DR.to_device(inp, dev)
    DR.run_round(d)
    ref = DR.outputs_to_host(d)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            DR.run_round(d)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        d.x.fill_(-7)
        d.next_tok.fill_(-7)
        d.ws_sample.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        got = DR.outputs_to_host(d)
        for k in ref:
            np.testing.assert_array_equal(np.asarray(ref[k]), np.asarray(got[k]), err_msg=f"{k} replay {rep}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_round_equals_four_calls(dev, dtype):
    """The round's fused draft-and-confidence call and the four separate
    calls (sample, confidence, schedule, verify) give the same outputs bit
    for bit; the sweep events of the fused call bracket a positive time."""
    from semi_ar_draft_round_amd import binding as B
    from semi_ar_draft_round_amd import device_round as DR
    w = W.custom(f"fused_{dtype}_r40_g5_v3000", R=40, gamma=5, V=3000, r=256 if dtype == "bf16" else 64, d=128,
                 dtype=dtype, seed=47, temperatures=True)
    inp = W.make_inputs(w)
    say(f"[parity] {w.name}")
    d = DR.to_device(inp, dev)
    DR.run_round_four_calls(d)
    ref = DR.outputs_to_host(d)
    timer = B.SweepTimer()
    DR.sample_conf(d, timer=timer)
    DR.schedule(d)
    DR.verify(d)
    out = DR.outputs_to_host(d)
    assert timer.elapsed_ms() > 0
    assert int(d.status.cpu()[0]) == 0
    for k in ("x", "lse", "logit", "c", "z", "ell", "n_acc", "next_tok"):
        np.testing.assert_array_equal(out[k], ref[k], err_msg=k)
    assert out["A"] == ref["A"] and out["theta_best"] == ref["theta_best"]


def test_sampling_kernel_choice(dev):
    """The sampling call names the kernel it runs: W2t held on chip up to
    eight tiles per compute unit, ten for a single block of 32 requests at
    r = 256 (one grid barrier per block of 32 requests from 65 to 1024
    requests, one per position up to 64), streamed otherwise."""
    from semi_ar_draft_round_amd import binding as B
    bf, f32 = torch.bfloat16, torch.float32
    assert B.dspark_markov_sample_kernel(bf, 128, 16, 129280, 256).startswith("sample_steps_pipe")
    assert B.dspark_markov_sample_kernel(bf, 256, 16, 129280, 256).startswith("sample_steps_pipe")
    assert B.dspark_markov_sample_kernel(bf, 65, 16, 129280, 256).startswith("sample_steps_pipe")
    assert B.dspark_markov_sample_kernel(bf, 1024, 2, 640, 64).startswith("sample_steps_pipe")
    assert B.dspark_markov_sample_kernel(bf, 1025, 2, 640, 64).startswith("sample_steps_wide")
    assert B.dspark_markov_sample_kernel(bf, 64, 16, 129280, 256).startswith("sample_steps_res")
    assert B.dspark_markov_sample_kernel(bf, 1, 16, 4096, 128).startswith("sample_steps_res")
    assert B.dspark_markov_sample_kernel(bf, 128, 16, 151936, 256).startswith("sample_steps_wide")
    assert B.dspark_markov_sample_kernel(bf, 1, 16, 151936, 256).startswith("sample_steps_res")
    assert B.dspark_markov_sample_kernel(bf, 32, 16, 163840, 256).startswith("sample_steps_res")
    assert B.dspark_markov_sample_kernel(bf, 32, 16, 163841, 256).startswith("sample_steps_wide")
    assert B.dspark_markov_sample_kernel(bf, 33, 16, 151936, 256).startswith("sample_steps_wide")
    assert B.dspark_markov_sample_kernel(bf, 1, 16, 151936, 128).startswith("sample_steps_wide")
    assert B.dspark_markov_sample_kernel(f32, 4, 3, 1000, 64).startswith("sample_step_f32")
    assert B.dspark_markov_sample_kernel(bf, 128, 16, 129280, 96) is None
