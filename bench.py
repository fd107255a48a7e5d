#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X.

Default workload (the metric's configuration): dense-vocab verify -- 64
requests, block K=7, vocabulary 151,936, bf16 logits, full-block windows,
temperature 1. One step is one pass of the whole path over that batch:
survival products + window selection (a flat step-time table makes every
window the full block), ragged pack, and the rejection verify (row statistics,
decisions, residual sums, inverse-CDF draws). Inputs are generated on the host
from fixed seeds, copied to HBM before timing, and reused for every step (the
Philox round changes per step).

Other workloads (--workload):
  scheduled-verify  confidence-scheduled ragged verify (256 x 16, mixed easy/hard streams)
  markov-chain      Markov-head greedy chain (256 requests x 16 steps, rank 256)
  pctree            PCTree expansion (128 x depth 16, k=4, F=16, N=64) + greedy tree verify
  cycle             sampled Markov draft (256 x 16, emitting its bf16 rows) -> confidence head -> schedule
                    -> pack -> verify
  copy              1 GiB device copy (reference for scaling HBM counters)

Prints ONE JSON line. `roofline` covers the dominant kernel of the workload,
timed with HIP events recorded by libdsp on the launch stream during the timed
region; `cpu_baseline` times the CPU oracle on a bounded sample of the same
batch (rank 0, N=1 only).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense-verify",
                    choices=["dense-verify", "scheduled-verify", "markov-chain", "pctree", "cycle", "copy"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prof-all", action="store_true", help="time every kernel with events (diagnostic)")
    return ap.parse_args()


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profiles(kernel_file, kernel_name, workload):
    """HBM bytes per launch measured with rocprofv3 counters, if taken on the current source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{workload}:{kernel_name}")
    if not rec:
        return None
    src = os.path.join(ROOT, "block_drafting_verification_amd", "csrc", kernel_file)
    if rec.get("source_sha") != _sha(src):
        return None
    return rec.get("bytes_per_launch")


def run_phases(make_step, steps, warmup, dominant, prof_all=False):
    """Time a step eagerly (HIP events around the dominant kernels only) and as a replayed HIP graph.

    make_step(stream) returns a zero-argument callable issuing one step of
    prepared libdsp calls on `stream`. Returns (eager_s, graph_s, kernels).
    """
    import torch
    import block_drafting_verification_amd as dsp
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step = make_step(s)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        dsp.prof_reset()
        dsp.prof_enable(True, kernels=None if prof_all else dominant)
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        eager = time.perf_counter() - t0
        dsp.prof_enable(False)
        kern = {}
        for name in dsp.KERNELS:
            ms, n = dsp.prof_query(name)
            if n:
                kern[name] = dict(avg_us=1000.0 * ms / n, launches=n)
        dsp.prof_reset()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        graph = time.perf_counter() - t0
    return eager, graph, kern


def cpu_oracle_verify(c, windows, budget_s, temperature=1.0):
    """Time the oracle on whole requests of the batch until the budget is spent."""
    import numpy as np
    import workloads
    from oracle import verify as ov
    R, K = c["R"], c["K"]
    done_tokens, done_req, passes = 0, 0, 0
    w0, c0 = time.perf_counter(), time.process_time()
    while time.perf_counter() - w0 < budget_s:
        for i in range(R):
            n = int(windows[i])
            t = workloads.values(c["t"][i, :n + 1], c["dtype"]).astype(np.float64)
            d = workloads.values(c["d"][i:i + 1], c["dtype"]).astype(np.float64)
            ov.verify_chain(t, np.array([0, n + 1]), d, c["x"][i:i + 1], temperature, seed=0, rnd=passes,
                            req_id=[i])
            done_tokens += n
            done_req += 1
            if time.perf_counter() - w0 > budget_s:
                break
        passes += 1
    wall = time.perf_counter() - w0
    cpu = time.process_time() - c0
    return dict(value=done_tokens / wall, unit="verified draft tokens/s", cores=max(1, round(cpu / wall)),
                kind="oracle", sample=f"{done_req} request-verifies over {passes} pass(es) of the {R}-request "
                                      f"batch ({done_tokens} verified draft tokens, {wall:.1f} s wall)")


def bench_verify(args, which):
    import numpy as np
    import torch
    import block_drafting_verification_amd as dsp
    import workloads

    dev = torch.device("cuda", 0)
    c = workloads.dense_verify() if which == "dense-verify" else workloads.scheduled_verify()
    R, K, V = c["R"], c["K"], c["V"]

    def gpu(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    conf, cost, anchors, x = gpu(c["conf"]), gpu(c["cost"]), gpu(c["anchors"]), gpu(c["x"])
    drf = bf16(c["d"])
    # windows are a deterministic function of the confidences: compute them once to lay out the
    # packed target logits (they stand in for the target forward over the packed buffer)
    w0 = dsp.schedule_windows(conf, cost)["windows"].cpu().numpy()
    if which == "dense-verify":
        tgt = bf16(c["t"].reshape(R * (K + 1), V))
    else:
        tgt = bf16(np.concatenate([c["t"][i, :w0[i] + 1] for i in range(R)]))
    max_rows = tgt.shape[0]
    rnd = torch.zeros(1, dtype=torch.int64, device=dev)
    ops = {}

    def make_step(stream):
        # the scheduler and the pack in one call (one launch: the selection workgroup packs)
        sch = dsp.schedule_pack(conf, cost, anchors, x, want_survival=False, stream=stream, prepare=True)
        pk = sch
        ver = dsp.verify_rejection(tgt, pk.outputs["cu_seqlens"], x, drf=drf, temperature=1.0, seed=0,
                                   round_dev=rnd, max_rows=max_rows, row_req=pk.outputs["row_req"],
                                   row_pos=pk.outputs["row_pos"], stream=stream, prepare=True)
        ops.update(sch=sch, pk=pk, ver=ver)

        def step():  # the verify call advances the device-side Philox round itself
            sch()
            ver()
        return step

    eager, graph, kern = run_phases(make_step, args.steps, args.warmup, ["VERIFY_STATS"], args.prof_all)
    elapsed = min(eager, graph)
    so = ops["sch"].outputs
    vo = ops["ver"].outputs
    assert int(ops["pk"].outputs["status"].item()) == 0 and int(vo["status"].item()) == 0, \
        "device status flagged a fault"
    win = so["windows"].cpu().numpy()
    assert np.array_equal(win, w0)
    N = int(win.sum())
    T_rows = R + N
    acc = vo["accepted_len"].cpu().numpy()
    bytes_stats = (T_rows + N) * V * 2
    st = kern["VERIFY_STATS"]["avg_us"]
    achieved = bytes_stats / (st * 1e-6) / 1e9
    traffic = traffic_from_profiles("verify.hip", "verify_stats", which)
    res = dict(
        metric="verified draft tokens/sec", value=N * args.steps / elapsed, unit="tokens/s",
        n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=1000.0 * elapsed / args.steps,
        higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
        data="synthetic (seeded N(0,3) logits with 1% +8 boosts; draft = target + Gaussian noise)",
        config=dict(workload=("dense-vocab verify: 64 requests, K=7, V=151936, bf16, full-block windows, T=1"
                              if which == "dense-verify" else
                              "confidence-scheduled ragged verify: 256 requests, K=16, V=151936, bf16, "
                              "additive cost 1+0.05n, compact windows, T=1"),
                    requests=R, block=K, vocab=V, logits_dtype="bf16",
                    arithmetic="fp32 per element (exp2), fp64 sums and decisions",
                    verified_drafts_per_step=N, packed_rows=T_rows, mean_accepted=float(acc.mean())),
        roofline=dict(kernel="verify_stats", bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=achieved / PEAK_HBM_GBS, traffic=traffic, algorithmic_bytes=bytes_stats,
                      avg_us=st),
        kernels=kern,
        timing=dict(graph_ms_per_step=1000.0 * graph / args.steps, eager_ms_per_step=1000.0 * eager / args.steps,
                    value_from="graph" if graph <= eager else "eager"),
    )
    res["roofline"]["read_ref"] = read_reference(tgt, drf)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_oracle_verify(c, win, args.cpu_seconds)
    return res


def read_reference(*tensors, reps=10):
    """Achievable read rate on this machine over the same buffers, outside the timed step: the
    library's streaming-read probe (plain 16-byte loads) over each; a second denominator beside
    the HBM peak."""
    import torch
    import block_drafting_verification_amd as dsp
    nbytes = sum(t.numel() * t.element_size() for t in tensors)
    sink = torch.zeros(1, dtype=torch.int32, device=tensors[0].device)
    for t in tensors:
        dsp.stream_read(t, sink)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        for t in tensors:
            dsp.stream_read(t, sink)
    b.record()
    b.synchronize()
    sec = a.elapsed_time(b) / 1e3 / reps
    return dict(GBps=nbytes / sec / 1e9, bytes=nbytes, frac_of_peak=nbytes / sec / 1e9 / PEAK_HBM_GBS,
                method="streaming-read probe over the same target and draft logits")


def bench_markov(args):
    import numpy as np
    import torch
    import block_drafting_verification_amd as dsp
    import workloads

    dev = torch.device("cuda", 0)
    c = workloads.markov_chain()
    R, B, V, r = c["R"], c["B"], c["V"], c["rank"]

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    L, U, Wt = bf16(c["L"]), bf16(c["U"]), bf16(np.ascontiguousarray(c["W"].T))
    a = torch.from_numpy(c["anchors"]).to(dev)
    def make_step(stream):
        return dsp.draft_markov_step(L, U, Wt, a, stream=stream, prepare=True)

    eager, graph, kern = run_phases(make_step, args.steps, args.warmup, ["MARKOV_GEMM", "MARKOV_MERGE"],
                                    args.prof_all)
    elapsed = min(eager, graph)
    g = kern["MARKOV_GEMM"]["avg_us"]
    # one launch reads the step's base logits L, the previous tokens' rows of U and all of Wt
    bytes_launch = R * V * 2 + R * r * 2 + V * r * 2
    flops_launch = 2.0 * R * r * V
    res = dict(
        metric="drafted tokens/sec", value=R * B * args.steps / elapsed, unit="tokens/s", n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=1000.0 * elapsed / args.steps, higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload="Markov-head greedy chain: 256 requests, 16 steps, V=151936, rank 256"),
        roofline=dict(kernel="markov_gemm", bound="hbm", achieved=bytes_launch / (g * 1e-6) / 1e9,
                      peak=PEAK_HBM_GBS, unit="GB/s", frac=bytes_launch / (g * 1e-6) / 1e9 / PEAK_HBM_GBS,
                      traffic=traffic_from_profiles("markov.hip", "markov_gemm", "markov-chain"),
                      mfma_tflops=flops_launch / (g * 1e-6) / 1e12,
                      mfma_frac=flops_launch / (g * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, avg_us=g),
        kernels=kern,
        timing=dict(graph_ms_per_step=1000.0 * graph / args.steps, eager_ms_per_step=1000.0 * eager / args.steps))
    if not args.no_cpu_baseline:
        from oracle import markov as om
        L32 = workloads.bf16_bits_to_f32(c["L"][:4])
        U32, W32 = workloads.bf16_bits_to_f32(c["U"]), workloads.bf16_bits_to_f32(c["W"])
        t0 = time.perf_counter()
        c0 = time.process_time()
        om.chain(L32, U32, W32, c["anchors"][:4])
        wall = time.perf_counter() - t0
        res["cpu_baseline"] = dict(value=4 * B / wall, unit="drafted tokens/s",
                                   cores=max(1, round((time.process_time() - c0) / wall)), kind="oracle",
                                   sample=f"4 of {R} requests, all {B} steps")
    return res


def bench_tree(args):
    import numpy as np
    import torch
    import block_drafting_verification_amd as dsp
    import workloads

    dev = torch.device("cuda", 0)
    c = workloads.pctree()
    R, D, V, r = c["R"], c["B"], c["V"], c["rank"]
    k, F, N = c["topk"], c["frontier"], c["topN"]

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    L, U, Wt = bf16(c["L"]), bf16(c["U"]), bf16(np.ascontiguousarray(c["W"].T))
    a = torch.from_numpy(c["anchors"]).to(dev)
    tgt = bf16(c["target"].reshape(R * (N + 1), V))
    cu = torch.arange(R + 1, dtype=torch.int32, device=dev) * (N + 1)
    def make_step(stream):
        te = dsp.tree_expand(L, U, Wt, a, k, F, N, stream=stream, prepare=True)
        tv = dsp.verify_rejection(tgt, cu, te.outputs["node_token"], parent=te.outputs["node_parent"],
                                  temperature=0.0, want_probs=False, stream=stream, prepare=True)

        def step():
            te()
            tv()
        return step

    eager, graph, kern = run_phases(make_step, args.steps, args.warmup, ["TREE_GEMM", "VERIFY_STATS"],
                                    args.prof_all)
    elapsed = min(eager, graph)
    f = []
    prev = 1
    for _ in range(D):
        prev = min(F, k * prev)
        f.append(prev)
    parents = R * (1 + sum(f[:-1]))
    flops = 2.0 * parents * r * V
    g = kern["TREE_GEMM"]
    gemm_total_us = g["avg_us"] * g["launches"] / args.steps
    res = dict(
        metric="tree nodes/sec", value=R * N * args.steps / elapsed, unit="nodes/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=1000.0 * elapsed / args.steps, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload="PCTree expansion + greedy tree verify: 128 requests, depth 16, V=129280, rank 256, "
                             "k=4, F=16, N=64"),
        roofline=dict(kernel="tree_gemm (all depths)", bound="mfma",
                      achieved=flops / (gemm_total_us * 1e-6) / 1e12, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                      frac=flops / (gemm_total_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, traffic=None,
                      gemm_us_per_step=gemm_total_us),
        kernels=kern,
        timing=dict(graph_ms_per_step=1000.0 * graph / args.steps, eager_ms_per_step=1000.0 * eager / args.steps))
    vs = kern["VERIFY_STATS"]["avg_us"]
    res["tree_verify"] = dict(bytes=R * (N + 1) * V * 2, avg_us=vs,
                              GBps=R * (N + 1) * V * 2 / (vs * 1e-6) / 1e9)
    return res


def bench_cycle(args):
    """Draft -> confidence head -> schedule -> pack -> verify, one HIP graph per step (the
    pages' cycle).

    The Markov head samples 16 positions for 256 requests and emits its bf16 rows (the
    verify's q); the confidence head (hidden size 4096, sequential temperatures) gives the
    per-position confidences from which the scheduler picks windows; the pack lays
    out the verify buffer; the verify checks the windows against target rows laid out in
    packed order at setup (they stand in for the target forward, which is not part of the
    method and is not timed).
    """
    import numpy as np
    import torch
    import block_drafting_verification_amd as dsp
    import workloads

    dev = torch.device("cuda", 0)
    c = workloads.cycle_case(256, 16, workloads.V_QWEN3, 256, seed=1006)
    R, K, V, r = c["R"], c["K"], c["V"], c["rank"]

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    L, U, Wt = bf16(c["L"]), bf16(c["U"]), bf16(np.ascontiguousarray(c["W"].T))
    a = torch.from_numpy(c["anchors"]).to(dev)
    hd = workloads.cycle_head_inputs(c)
    hh, hw = bf16(hd["h"]), bf16(hd["w"])
    temps = torch.from_numpy(hd["temps"]).to(dev)
    cost = torch.from_numpy(c["cost"]).to(dev)
    conf0 = dsp.confidence_head(hh, hw, hd["bias"], temps)["conf"]
    w0 = dsp.schedule_windows(conf0, cost)["windows"].cpu().numpy()
    tgt = bf16(workloads.cycle_target(c, w0))
    rd = torch.zeros(1, dtype=torch.int64, device=dev)
    ops = {}

    def make_step(stream):
        dr = dsp.draft_markov_sample(L, U, Wt, a, 1.0, seed=0, round_dev=rd, stream=stream, prepare=True)
        ch = dsp.confidence_head(hh, hw, hd["bias"], temps, stream=stream, prepare=True)
        sch = dsp.schedule_pack(ch.outputs["conf"], cost, a, dr.outputs["y"], want_survival=False, stream=stream,
                                prepare=True)
        pk = sch
        ver = dsp.verify_rejection(tgt, pk.outputs["cu_seqlens"], dr.outputs["y"], drf=dr.outputs["z"],
                                   temperature=1.0, seed=0, round_dev=rd, max_rows=tgt.shape[0],
                                   row_req=pk.outputs["row_req"], row_pos=pk.outputs["row_pos"],
                                   want_probs=False, stream=stream, prepare=True)
        ops.update(dr=dr, ch=ch, sch=sch, pk=pk, ver=ver)

        def step():
            dr()
            ch()
            sch()
            ver()
        return step

    eager, graph, kern = run_phases(make_step, args.steps, args.warmup, ["MARKOV_GEMM", "MARKOV_MERGE",
                                                                          "VERIFY_STATS"], args.prof_all)
    elapsed = min(eager, graph)
    for k in ("dr", "ch", "pk", "ver"):
        assert int(ops[k].outputs["status"].item()) == 0, "device status flagged a fault"
    win = ops["sch"].outputs["windows"].cpu().numpy()
    assert np.array_equal(win, w0)
    N = int(win.sum())
    acc = ops["ver"].outputs["accepted_len"].cpu().numpy()
    g = kern["MARKOV_GEMM"]["avg_us"]
    # one sampled step reads L's rows, the previous tokens' U rows and Wt, and writes the bf16 rows
    bytes_launch = R * V * 2 + R * r * 2 + V * r * 2 + R * V * 2
    res = dict(
        metric="verified draft tokens/sec", value=N * args.steps / elapsed, unit="tokens/s", n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=1000.0 * elapsed / args.steps, higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="bf16",
        data="synthetic (Markov-head inputs; target rows = draft base logits + per-request noise, packed order)",
        config=dict(workload="draft -> confidence head -> schedule -> pack -> verify cycle: 256 requests, "
                             "16 sampled drafts, V=151936, rank 256, hidden 4096, T=1, additive cost 1+0.05n",
                    requests=R, block=K, vocab=V, drafted_per_step=R * K, verified_drafts_per_step=N,
                    packed_rows=R + N, mean_accepted=float(acc.mean()),
                    drafted_tokens_per_s=R * K * args.steps / elapsed),
        roofline=dict(kernel="markov_gemm (sampled, emits bf16 rows)", bound="hbm",
                      achieved=bytes_launch / (g * 1e-6) / 1e9, peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=bytes_launch / (g * 1e-6) / 1e9 / PEAK_HBM_GBS,
                      traffic=traffic_from_profiles("markov.hip", "markov_gemm", "cycle"),
                      algorithmic_bytes=bytes_launch, avg_us=g),
        kernels=kern,
        timing=dict(graph_ms_per_step=1000.0 * graph / args.steps, eager_ms_per_step=1000.0 * eager / args.steps))
    return res


def bench_copy(args):
    """Plain device-to-device copy of a 1 GiB buffer: the reference for scaling HBM counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    return dict(metric="copy bandwidth", value=2 * n / dt / 1e9, unit="GB/s (read + write)", bytes_read=n,
                bytes_written=n, steps=args.steps, ms_per_step=dt * 1e3)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the path is not "
              "sharded across GPUs.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.workload == "copy":
        res = bench_copy(args)
    elif args.workload in ("dense-verify", "scheduled-verify"):
        res = bench_verify(args, args.workload)
    elif args.workload == "markov-chain":
        res = bench_markov(args)
    elif args.workload == "cycle":
        res = bench_cycle(args)
    else:
        res = bench_tree(args)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
