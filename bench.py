"""Benchmark: one DSpark draft-and-verify round (the draft with its
confidences -> schedule -> verify) on one MI355X, as drafted tokens per
second.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one round of the whole path over one batch of synthetic inputs
already resident in HBM, replayed from a captured HIP graph.  Two input sets
(different logits, hidden states and noise; the same weights) alternate
between steps so that a step cannot be served from the previous step's
cache lines.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix cores
METRIC = "drafted tokens/s (sample+schedule+verify) at R=128 γ=16 V=129280; % HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the sources the sampling launch is built from."""
    h = hashlib.sha256()
    for rel in ("semi_ar_draft_round_amd/csrc/sample.hip", "semi_ar_draft_round_amd/csrc/sample_res.hip",
                "semi_ar_draft_round_amd/csrc/sample_pipe.hip",
                "semi_ar_draft_round_amd/csrc/sample_common.hpp", "semi_ar_draft_round_amd/csrc/bias_tile.hpp",
                "semi_ar_draft_round_amd/csrc/wide_tile.hpp", "semi_ar_draft_round_amd/csrc/common.hpp",
                "semi_ar_draft_round_amd/csrc/sample_keys.hpp", "semi_ar_draft_round_amd/csrc/rnn_head.hpp",
                "include/dspark.h"):
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(rel.encode() + fh.read())
    return h.hexdigest()[:16]


def sample_bytes_per_position(w) -> int:
    """Algorithmic HBM bytes of one sampling position: the U_k slice of every
    request and the whole W2t (the bias product's operand).  The chunk
    Gumbels, which a counter-based generator would make in registers, are
    not counted (noise_bytes_per_position)."""
    return w.R * w.V * 2 + w.r * w.V * 2


def noise_bytes_per_position(w) -> int:
    """HBM bytes of one position's chunk Gumbels as this harness stores them."""
    return w.R * w.n_chunks * 4


def _oracle_rounds(inps, n_req: int, min_seconds: float, max_rounds: int):
    """Free-running oracle rounds over n_req requests: (rounds, requests, seconds)."""
    import numpy as np
    from oracle.round import run_round
    w = inps[0].w
    idx = np.arange(min(n_req, w.R))
    done, dt = 0, 0.0
    while done < max_rounds and (dt < min_seconds or done == 0):
        t0 = time.perf_counter()
        run_round(inps[done % len(inps)], requests=idx)
        dt += time.perf_counter() - t0
        done += 1
    return done, len(idx), dt


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inps, n_req: int, min_seconds: float = 10.0, max_rounds: int = 8) -> dict:
    """The float64 oracle, free running, on a bounded sample of the same
    workload: n_req requests per round (the whole batch when n_req >= R),
    repeated over the input sets until at least min_seconds of CPU work;
    then a second, single-threaded run over a quarter of the requests."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threadpool_limits = None
        threads = 1
    w = inps[0].w
    done, nr, dt = _oracle_rounds(inps, n_req, min_seconds, max_rounds)
    part = "the whole batch" if nr == w.R else f"{nr} of {w.R} requests"
    rec = {"value": done * nr * w.gamma / dt, "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle",
           "sample": f"{done} free-running rounds of {part} (gamma={w.gamma}, V={w.V}): "
                     f"sample, confidence, schedule, verify; {dt:.1f} s of CPU work",
           "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count(), "blas_threads": int(threads)}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            d1, n1, t1 = _oracle_rounds(inps, max(1, min(n_req, w.R) // 4), min_seconds / 2, max_rounds)
        rec["single_thread"] = {"value": d1 * n1 * w.gamma / t1, "unit": "tokens/s",
                                "sample": f"{d1} rounds of {n1} of {w.R} requests, one thread; {t1:.1f} s"}
    return rec


def traffic_record(workload: str, kernel: str):
    """HBM traffic per sampling launch from committed rocprofv3 counter runs
    of the kernel in use, only if they were taken on the current sources."""
    tag = (kernel or "").split(":")[0].replace("sample_steps_", "")
    p = os.path.join(ROOT, "profiles", f"traffic_sample_steps_{tag}_{workload}.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


kEagerSkip = 60   # eager rounds run before the counted ones (about 25 ms of work)

# The other single-GPU bf16 workloads the bench line also reports.
OTHER_WORKLOADS = ("latency_r1_g16_v151936", "batch_r32_g16_v151936", "heavy_r128_g16_v129280",
                   "full_r256_g16_v129280_sts")


def measure_other(w, dev, steps):
    """The round (graph replays, two alternating input sets) and the
    persistent sampling launch (events over eager rounds) of one workload."""
    import numpy as np
    import torch
    from semi_ar_draft_round_amd import binding, workloads as W
    from semi_ar_draft_round_amd import device_round as DR
    t0 = time.perf_counter()
    rounds = [DR.to_device(W.make_inputs(w, round_index=i), dev) for i in range(2)]
    rounds[1].W1, rounds[1].W2t, rounds[1].w = rounds[0].W1, rounds[0].W2t, rounds[0].w
    for d in rounds:
        DR.run_round(d)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graphs = []
    for d in rounds:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                DR.run_round(d)
        torch.cuda.current_stream().wait_stream(stream)
        graphs.append(g)
    torch.cuda.synchronize()
    timers = [binding.SweepTimer() for _ in range(steps)]
    for i in range(len(timers) + kEagerSkip):
        d = rounds[i % 2]
        DR.sample_conf(d, timer=timers[i - kEagerSkip] if i >= kEagerSkip else None)
        DR.schedule(d)
        DR.verify(d)
    torch.cuda.synchronize()
    launch_us = float(np.mean([t.elapsed_ms() * 1e3 for t in timers]))
    for i in range(3):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        graphs[i % 2].replay()
    end.record()
    torch.cuda.synchronize()
    round_us = start.elapsed_time(end) / steps * 1e3
    kernel = binding.dspark_markov_sample_kernel(rounds[0].U.dtype, w.R, w.gamma, w.V, w.r)
    bytes_launch = sample_bytes_per_position(w) * w.gamma
    rec = {"round_us": round(round_us, 1), "tokens_per_s": round(w.R * w.gamma / (round_us * 1e-6), 1),
           "launch_us": round(launch_us, 1), "frac": round(bytes_launch / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "kernel": kernel.split(":")[0], "seconds": round(time.perf_counter() - t0, 1)}
    del graphs, rounds
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-requests", type=int, default=1 << 30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-modes", action="store_true",
                    help="skip timing the other modes (the production scheduler, greedy verification, the "
                         "analytic acceptance, the RNN-head draft, STS), e.g. for counter runs on the round")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the round and sampling-launch timings of the other bf16 workloads")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only copy a buffer of this many MiB a few times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: it measures one GPU's share of the hot path. "
              "Requests shard across GPUs with no exchange, so the per-GPU figure is the "
              "whole story; --gpus > 1 is not run.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        b = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_probe_mib} MiB three times")
        return
    from semi_ar_draft_round_amd import binding, workloads as W
    from semi_ar_draft_round_amd import device_round as DR

    binding.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = W.BY_NAME[args.workload or W.BENCH_WORKLOAD]
    log(f"[bench] workload {w.name}: drawing inputs")
    t0 = time.perf_counter()
    inps = [W.make_inputs(w, round_index=i) for i in range(2)]
    log(f"[bench] inputs drawn in {time.perf_counter() - t0:.1f} s; copying to {dev}")
    rounds = [DR.to_device(inps[0], dev, rnn=True)]
    d1 = DR.to_device(inps[1], dev, rnn=True)
    d1.W1, d1.W2t, d1.w = rounds[0].W1, rounds[0].W2t, rounds[0].w   # weights are shared
    d1.rnn["W"] = rounds[0].rnn["W"]
    rounds.append(d1)
    # the RNN head's table P (W's W1-row columns applied to every W1 row) is
    # made once per set of weights, as a server would at load time; the
    # rnn_prepare mode below times making it
    DR.rnn_prepare(rounds[0])
    d1.rnn["P"] = rounds[0].rnn["P"]
    torch.cuda.synchronize()

    # eager warm-up, then one captured graph per input set and per part
    for d in rounds:
        DR.run_round(d)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())

    def capture(fn, d):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                fn(d)
        torch.cuda.current_stream().wait_stream(stream)
        return g

    graphs = {name: [capture(fn, d) for d in rounds]
              for name, fn in (("round", DR.run_round), ("sample_conf", DR.sample_conf),
                               ("sample", DR.sample), ("confidence", DR.confidence), ("schedule", DR.schedule),
                               ("verify", DR.verify), ("schedule_production", DR.schedule_production),
                               ("verify_greedy", DR.verify_greedy), ("acceptance", DR.acceptance),
                               ("rnn_sample", DR.rnn_sample), ("rnn_prepare", DR.rnn_prepare))}
    # sequential temperature scaling on a held-out set of 65536 rollouts
    # (gamma = 16, 61 temperatures, 15 bins), captured the same way
    if not args.no_modes:
        zs, ns = W.make_rollouts(65536, w.gamma, 2.0)
        sts_in = (torch.tensor(zs, device=dev), torch.tensor(ns, device=dev),
                  torch.tensor(W.sts_grid(), device=dev))
        binding.dspark_sts_fit(*sts_in, 15)
        torch.cuda.synchronize()
        graphs["sts_fit"] = [capture(lambda _d: binding.dspark_sts_fit(*sts_in, 15), None)] * 2
    torch.cuda.synchronize()
    log("[bench] graphs captured")

    def timed(name, steps, warmup):
        gs = graphs[name]
        for i in range(warmup):
            gs[i % 2].replay()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            gs[i % 2].replay()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps       # ms per replay

    # the persistent sampling launch alone: eager rounds (the same calls as
    # the graph, the same alternation of input sets), with the sampling call
    # stamping two HIP events with that launch's start and end on its stream
    # (the first kEagerSkip rounds are not counted: after the idle spell of
    # graph capture the GPU's clocks take a few milliseconds of work to
    # settle); each counted round has its own event pair, read after the
    # last round, so the host never waits between rounds
    timers = [binding.SweepTimer() for _ in range(max(args.steps, 10))]
    for i in range(len(timers) + kEagerSkip):
        d = rounds[i % 2]
        DR.sample_conf(d, timer=timers[i - kEagerSkip] if i >= kEagerSkip else None)
        DR.schedule(d)
        DR.verify(d)
    torch.cuda.synchronize()
    sweeps = [t.elapsed_ms() * 1e3 for t in timers]
    sweep_us = float(np.mean(sweeps))
    log(f"[bench] persistent sampling launch: mean {sweep_us:.1f} us over {len(sweeps)} eager rounds "
        f"(min {min(sweeps):.1f}, max {max(sweeps):.1f})")
    # the round itself, timed after the eager rounds above: the GPU has then
    # been busy for a while, so its clocks have settled (after an idle spell
    # the first few rounds run several per cent slower)
    ms = timed("round", args.steps, args.warmup)
    log(f"[bench] round: {ms * 1e3:.1f} us")
    # the spread of single rounds, each bracketed by its own events (a second
    # pass after the timed region above, which alone gives `value`)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(args.steps, 20))]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        graphs["round"][i % 2].replay()
        e1.record()
    torch.cuda.synchronize()
    singles = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
    spread = [round(float(np.percentile(singles, q)), 1) for q in (10, 50, 90)]
    log(f"[bench] single rounds p10/p50/p90: {spread} us")
    # the round's three calls, each replayed on its own
    parts = {}
    for name in ("sample_conf", "schedule", "verify"):
        parts[name] = timed(name, max(args.steps, 10), 2) * 1e3
        log(f"[bench] {name}: {parts[name]:.1f} us")
    # the other modes, each timed on its own and outside the round: the
    # sampling call without and the confidence head as a call of its own, the
    # production (asynchronous) scheduler's two calls, greedy verification of
    # the round's drafts, the analytic acceptance of all its positions, the
    # draft with the RNN head (with its table P made beforehand), making P,
    # and the calibration fit
    modes = {}
    for name in () if args.no_modes else ("sample", "confidence", "schedule_production", "verify_greedy",
                                          "acceptance", "rnn_sample", "rnn_prepare", "sts_fit"):
        modes[name] = timed(name, max(args.steps, 10), 2) * 1e3
        log(f"[bench] {name}: {modes[name]:.1f} us")

    # outputs of the last replay of input set 0, as workload facts
    graphs["round"][0].replay()
    out = DR.outputs_to_host(rounds[0])
    value = w.R * w.gamma / (ms * 1e-3)

    # The dominant kernel is the persistent sampling launch over all gamma
    # positions.  Its algorithmic bytes: gamma x (U_k of every request + W2t).
    bytes_launch = sample_bytes_per_position(w) * w.gamma
    # the on-chip-reuse floor: W2 read once per launch instead of once per position
    bytes_model_b = bytes_launch - (w.gamma - 1) * w.r * w.V * 2
    achieved = bytes_launch / (sweep_us * 1e-6) / 1e9
    kernel = binding.dspark_markov_sample_kernel(rounds[0].U.dtype, w.R, w.gamma, w.V, w.r)
    traffic = traffic_record(w.name, kernel)
    # the bias product's work, for the matrix-core view of the same launch
    flops_launch = 2.0 * w.R * w.r * w.V * w.gamma
    tflops = flops_launch / (sweep_us * 1e-6) / 1e12
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": kernel,
                "mfma_bf16": {"achieved_tflops": round(tflops, 1), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                              "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                              "flops_per_launch": flops_launch},
                "bytes_per_launch": bytes_launch, "us_per_launch": round(sweep_us, 2),
                "noise_bytes_per_launch": noise_bytes_per_position(w) * w.gamma,
                "bytes_per_launch_w2_once": bytes_model_b,
                "frac_w2_once": round(bytes_model_b / (sweep_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "frac_traffic": None if traffic is None else
                round(traffic / (sweep_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "R": w.R, "gamma": w.gamma, "V": w.V, "r": w.r, "d": w.d,
                   "global_batch": w.R, "admitted": out["A"], "accepted": int(out["n_acc"].sum()),
                   "parallelism": "none (1 GPU)"},
        "round_us_p10_p50_p90": spread,
        "parts_us": {k: round(v, 2) for k, v in parts.items()},
        "modes_us": {k: round(v, 2) for k, v in modes.items()},
        "roofline": roofline,
    }
    # the other bf16 workloads, each on its own inputs (two sets, as above):
    # the sampling launch by its events over eager rounds and the round graph
    if not args.no_other_workloads:
        rec["other_workloads"] = {}
        for name in OTHER_WORKLOADS:
            if name == w.name:
                continue
            rec["other_workloads"][name] = measure_other(W.BY_NAME[name], dev, max(args.steps, 10))
            log(f"[bench] {name}: {rec['other_workloads'][name]}")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        rec["cpu_baseline"] = cpu_baseline(inps, args.cpu_requests)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
