#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X.

Default workload (the largest configuration that fits one GPU): the
confidence-scheduled ragged verify -- 256 requests, block K=16, vocabulary
151,936, bf16 logits, per-request draft noise scales from U(0.2, 2.0), per-position
confidences from a logistic model of the draft-target total-variation distance,
additive step-time table c(n) = 1 + 0.05 n. One step is one pass of the whole path
over that batch: survival products, window selection and the ragged pack (one
launch), then the rejection verify of the packed windows (row statistics,
decisions, residual sums, inverse-CDF draws). A sub-record times the static run
of the same data (every window the full block: 8,448 logit rows, 2.567 GB).

Other workloads (--workload):
  dense-verify      64 requests x K=7 x V=151,936, full-block windows
  markov-chain      Markov-head greedy chain (256 requests x 16 steps, rank 256)
  rnn-chain         RNN-head greedy chain (256 x 16, rank 256, backbone hidden size 4096)
  pctree            PCTree expansion (128 x depth 16, k=4, F=16, N=64) + greedy tree verify
  cycle             sampled Markov draft (256 x 16, emitting its bf16 rows) -> confidence head
                    -> schedule -> pack -> verify
  copy              1 GiB device copy (reference for scaling HBM counters)

Timing: inputs are resident in HBM before the timed region. Each timed step is
preceded (outside its timed interval) by a 512 MiB store pass over a scratch buffer,
so the 256 MB Infinity Cache and the L2s hold nothing of the step's inputs; the step
time is the sum of HIP-event intervals around the steps on their stream. The value
comes from replays of one captured HIP graph per step (or eager launches if faster).
`roofline` covers the dominant kernel, its per-launch time taken from HIP events
that libdsp attaches to each dispatch on the launch stream during the eager pass.
`cpu_baseline` times the CPU oracle (the plain fp64 numpy implementation) on a bounded
sample of the same batch, over worker processes on the host's cores; it runs before
the GPU is touched, so the workers are forked from a process with no GPU state.

Prints ONE JSON line.
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
FLUSH_BYTES = 512 << 20     # cache flush between timed steps (2x the Infinity Cache)


def flush_caches(scratch, i):
    """Outside the timed interval: a plain store pass over a buffer twice the Infinity
    Cache's size evicts what the step left there, then a read pass over the same buffer
    writes the store pass's dirty lines back, so the next step starts from cold caches
    holding clean lines only (otherwise the step's first kernels pay for writing back up
    to the whole cache of the flush's own data)."""
    scratch.fill_(i + 1)  # elementwise store kernel (nonzero: no memset path)
    scratch.sum()         # reduction: reads the buffer
MAX_CPU_WORKERS = 16        # host cores given to one GPU


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="scheduled-verify",
                    choices=["scheduled-verify", "dense-verify", "markov-chain", "rnn-chain", "pctree", "cycle", "copy"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall budget of the parallel oracle sample")
    ap.add_argument("--cpu-single-seconds", type=float, default=4.0, help="wall budget of the 1-core sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true", help="diagnostic: no cache flush between timed steps")
    ap.add_argument("--chain-persistent", action="store_true",
                    help="markov-chain: all 16 steps in one persistent launch (default: one launch per step)")
    ap.add_argument("--general-gemm", action="store_true",
                    help="diagnostic: the general GEMM kernel for every tree depth (default: the scheduled kernel "
                         "where it applies; outputs are bit-identical)")
    ap.add_argument("--l-layout", default="row-major", choices=["row-major", "token-major"],
                    help="chain workloads: base logits [R, B, V] (row-major) or [B, V, R] (token-major)")
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


# ---------------------------------------------------------------- CPU baseline (oracle)
# Worker processes are forked before this process touches the GPU; they inherit the
# workload arrays and the task function through _CTX and run numpy single-threaded.
_CTX = {}


def _worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def _worker_task(i):
    return _CTX["fn"](i)


def cpu_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(MAX_CPU_WORKERS, n))


def cpu_baseline(fn, items, budget_s, single_s, unit, sample_desc):
    """Time fn(item) -> work units over passes of `items` until the wall budget is spent:
    in parallel over worker processes, then on one core. Returns the cpu_baseline record."""
    import multiprocessing as mp
    _CTX["fn"] = fn
    workers = cpu_workers()
    ctx = mp.get_context("fork")
    done_units, done_items, passes = 0.0, 0, 0
    with ctx.Pool(workers, initializer=_worker_init) as pool:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            for u in pool.imap_unordered(_worker_task, items, chunksize=max(1, len(items) // (4 * workers))):
                done_units += u
                done_items += 1
            passes += 1
        wall = time.perf_counter() - t0
    _worker_init()
    one_units, one_items = 0.0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < single_s:
        one_units += fn(items[one_items % len(items)])
        one_items += 1
    one_wall = time.perf_counter() - t0
    return dict(value=done_units / wall, unit=unit, cores=workers, kind="oracle",
                sample=f"{sample_desc}: {done_items} items over {passes} pass(es) of {len(items)} "
                       f"({done_units:.0f} {unit.split('/')[0]}, {wall:.1f} s wall, {workers} worker processes)",
                single_core=dict(value=one_units / one_wall, unit=unit, cores=1,
                                 sample=f"{one_items} items, {one_wall:.1f} s wall"))


# ---------------------------------------------------------------- GPU timing
def run_phases(make_step, steps, warmup, dominant, do_flush=True):
    """Time a step eagerly (HIP events attached to every libdsp dispatch) and as a replayed
    HIP graph, each timed step preceded by a cache-flushing store pass outside its interval.

    make_step(stream) returns a zero-argument callable issuing one step of prepared libdsp
    calls on `stream`. Returns dict(eager_s, graph_s, warm_graph_s, kernels).
    """
    import torch
    import block_drafting_verification_amd as dsp
    s = torch.cuda.Stream()
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")

    def flush(i):
        if do_flush:
            flush_caches(scratch, i)

    def timed(body):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i, (a, b) in enumerate(ev):
            flush(i)
            a.record(s)
            body()
            b.record(s)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / 1e3

    with torch.cuda.stream(s):
        step = make_step(s)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        dsp.prof_reset()
        dsp.prof_enable(True)
        eager = timed(step)
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
        graph = timed(g.replay)
        # context only: back-to-back replays with no flush (caches warm)
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        warm = time.perf_counter() - t0
    for k in dominant:
        assert k in kern, f"no timed launch of {k}"
    return dict(eager_s=eager, graph_s=graph, warm_graph_s=warm, kernels=kern)


def timing_record(ph, steps):
    elapsed = min(ph["eager_s"], ph["graph_s"])
    return elapsed, dict(graph_ms_per_step=1000.0 * ph["graph_s"] / steps,
                         eager_ms_per_step=1000.0 * ph["eager_s"] / steps,
                         warm_graph_ms_per_step=1000.0 * ph["warm_graph_s"] / steps,
                         value_from="graph" if ph["graph_s"] <= ph["eager_s"] else "eager",
                         cache_flush=f"{FLUSH_BYTES >> 20} MiB store pass, then a read pass over it, before each "
                                     "timed step")


def hbm_roofline(kernel, algo_bytes, avg_us, traffic):
    ach = algo_bytes / (avg_us * 1e-6) / 1e9
    r = dict(kernel=kernel, bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s", frac=ach / PEAK_HBM_GBS,
             traffic=traffic, algorithmic_bytes=algo_bytes, avg_us=avg_us)
    if traffic:
        r["traffic_over_algorithmic"] = traffic / algo_bytes
    return r


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


def _bf16(dev, bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def _chain_l(dev, bits, args):
    """Base logits [R, B, V] on the GPU, row-major or (a [B, V, R] buffer) token-major."""
    import numpy as np
    if args.l_layout == "row-major":
        return _bf16(dev, bits)
    return _bf16(dev, np.transpose(bits, (1, 2, 0))).permute(2, 0, 1)


def _gpu(dev, a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


# ---------------------------------------------------------------- verify workloads
def verify_data(which):
    import numpy as np
    import workloads
    from oracle import schedule as osch
    c = workloads.dense_verify() if which == "dense-verify" else workloads.scheduled_verify()
    # the windows are a deterministic function of the confidences: the oracle's gives the
    # layout of the packed target rows (which stand in for the target forward over the buffer)
    c["w0"] = osch.schedule_windows(c["conf"], c["cost"])["windows"].astype(np.int64)
    return c


def verify_cpu(c, args):
    import numpy as np
    import workloads
    from oracle import verify as ov
    win = c["w0"]

    def one(i):
        n = int(win[i])
        t = workloads.values(c["t"][i, :n + 1], c["dtype"])
        d = workloads.values(c["d"][i:i + 1], c["dtype"])
        ov.verify_chain(t, np.array([0, n + 1]), d, c["x"][i:i + 1], 1.0, seed=0, rnd=0, req_id=[i])
        return n
    return cpu_baseline(one, list(range(c["R"])), args.cpu_seconds, args.cpu_single_seconds,
                        "verified draft tokens/s", "oracle verify of whole requests of the batch (its windows)")


def bench_verify(args, which, c, cpu):
    import numpy as np
    import torch
    import block_drafting_verification_amd as dsp

    dev = torch.device("cuda", 0)
    R, K, V = c["R"], c["K"], c["V"]
    w0 = c["w0"]
    conf, cost, anchors, x = _gpu(dev, c["conf"]), _gpu(dev, c["cost"]), _gpu(dev, c["anchors"]), _gpu(dev, c["x"])
    drf = _bf16(dev, c["d"])
    # the packed target rows at the front of a buffer sized for the largest batch, R x (K+1)
    # rows: the step is captured once with max_rows = R x (K+1), as a caller that learns the
    # packed total only on the device would (its kernels skip the rows past that total)
    max_rows = R * (K + 1)
    if which == "dense-verify":
        tgt = _bf16(dev, c["t"].reshape(max_rows, V))
    else:
        tgt = torch.zeros(max_rows, V, dtype=torch.bfloat16, device=dev)
        packed = _bf16(dev, np.concatenate([c["t"][i, :w0[i] + 1] for i in range(R)]))
        tgt[:packed.shape[0]].copy_(packed)
        del packed
    rnd = torch.zeros(1, dtype=torch.int64, device=dev)
    ops = {}

    def make_step(stream):
        # the scheduler and the pack in one call (one launch: the selection workgroup packs)
        sch = dsp.schedule_pack(conf, cost, anchors, x, want_survival=False, stream=stream, prepare=True)
        ver = dsp.verify_rejection(tgt, sch.outputs["cu_seqlens"], x, drf=drf, temperature=1.0, seed=0,
                                   round_dev=rnd, max_rows=max_rows, row_req=sch.outputs["row_req"],
                                   row_pos=sch.outputs["row_pos"], stream=stream, prepare=True)
        ops.update(sch=sch, ver=ver)

        def step():  # the verify call advances the device-side Philox round itself
            sch()
            ver()
        return step

    ph = run_phases(make_step, args.steps, args.warmup, ["VERIFY_STATS"], not args.no_flush)
    elapsed, timing = timing_record(ph, args.steps)
    kern = ph["kernels"]
    so, vo = ops["sch"].outputs, ops["ver"].outputs
    assert int(so["status"].item()) == 0 and int(vo["status"].item()) == 0, "device status flagged a fault"
    win = so["windows"].cpu().numpy()
    assert np.array_equal(win, w0)
    N = int(win.sum())
    T_rows = R + N
    acc = vo["accepted_len"].cpu().numpy()
    bytes_stats = (T_rows + N) * V * 2
    wl = ("dense-vocab verify: 64 requests, K=7, V=151936, bf16, full-block windows, T=1"
          if which == "dense-verify" else
          "confidence-scheduled ragged verify: 256 requests, K=16, V=151936, bf16, TV-logistic confidences, "
          "additive cost 1+0.05n, compact windows, T=1")
    res = dict(
        metric="verified draft tokens/sec", value=N * args.steps / elapsed, unit="tokens/s",
        n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=1000.0 * elapsed / args.steps,
        higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
        data="synthetic (seeded N(0,3) logits with 1% +8 boosts; draft = target + Gaussian noise)",
        config=dict(workload=wl, requests=R, block=K, vocab=V, logits_dtype="bf16",
                    arithmetic="fp32 per element (exp2), fp64 sums and decisions",
                    verified_drafts_per_step=N, packed_rows=T_rows, captured_rows=max_rows,
                    mean_accepted=float(acc.mean()),
                    window_histogram=np.bincount(win, minlength=K + 1).tolist()),
        roofline=hbm_roofline("verify_stats", bytes_stats, kern["VERIFY_STATS"]["avg_us"],
                              traffic_from_profiles("verify.hip", "verify_stats", which)),
        kernels=kern, timing=timing)
    res["roofline"]["read_ref"] = read_reference(tgt, drf)
    if which == "scheduled-verify":
        res["static"] = bench_static(args, c, dev, drf, x)
        res["known_total"] = bench_tiering(args, c, dev, tgt, drf, x, conf, cost, anchors)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    return res


ROW_TIERS = [256, 320, 384, 512, 640, 768, 1024, 1536, 2048, 3072, 4352]


def bench_tiering(args, c, dev, tgt, drf, x, conf, cost, anchors):
    """The same step when the host learns the packed total before the verify, two ways:
    one graph captured with max_rows = the packed total (an upper bound on what a host
    that knows it gets), and one verify graph per row tier replayed by the tier the pack
    wrote (SGLang article, "Ragged verify"), which costs a read-back of that tier and a
    wait before the replay. tgt holds the packed rows at its front."""
    import torch
    import block_drafting_verification_amd as dsp
    R = c["R"]
    w0 = c["w0"]
    T = int(w0.sum()) + R
    N = int(w0.sum())
    out = {}

    # (a) one graph sized to the packed total
    rnd = torch.zeros(1, dtype=torch.int64, device=dev)

    def make_step(stream):
        sch = dsp.schedule_pack(conf, cost, anchors, x, want_survival=False, stream=stream, prepare=True)
        ver = dsp.verify_rejection(tgt, sch.outputs["cu_seqlens"], x, drf=drf, temperature=1.0, seed=0,
                                   round_dev=rnd, max_rows=T, row_req=sch.outputs["row_req"],
                                   row_pos=sch.outputs["row_pos"], stream=stream, prepare=True)

        def step():
            sch()
            ver()
        return step

    ph = run_phases(make_step, args.steps, args.warmup, ["VERIFY_STATS"], not args.no_flush)
    out["exact_size_graph"] = dict(ms_per_step=1000.0 * ph["graph_s"] / args.steps,
                                   value=N * args.steps / ph["graph_s"], max_rows=T,
                                   verify_stats_us=ph["kernels"]["VERIFY_STATS"]["avg_us"])

    # (b) one verify graph per tier, chosen from the pack's tier
    s = torch.cuda.Stream()
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    rnd2 = torch.zeros(1, dtype=torch.int64, device=dev)
    with torch.cuda.stream(s):
        sch = dsp.schedule_pack(conf, cost, anchors, x, want_survival=False, tiers=ROW_TIERS, stream=s,
                                prepare=True)
        shared = {"status": torch.zeros(1, dtype=torch.int32, device=dev)}

        def make(tier):
            v = dsp.verify_rejection(tgt, sch.outputs["cu_seqlens"], x, drf=drf, temperature=1.0, seed=0,
                                     round_dev=rnd2, max_rows=tier, row_req=sch.outputs["row_req"],
                                     row_pos=sch.outputs["row_pos"], out=shared, status=shared["status"],
                                     stream=s, prepare=True)
            shared.update({k: t for k, t in v.outputs.items() if t is not None})
            return v

        g_sch = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_sch, stream=s):
            sch()
        tg = dsp.TierGraphs(ROW_TIERS, make, stream=s)
        tt = sch.outputs["total_and_tier"]
        for _ in range(args.warmup):
            g_sch.replay()
            tg.replay(tt)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        tier = None
        for i, (a, b) in enumerate(ev):
            if not args.no_flush:
                flush_caches(scratch, i)
            a.record(s)
            g_sch.replay()
            tier = tg.replay(tt)
            b.record(s)
        torch.cuda.synchronize()
        sec = sum(a.elapsed_time(b) for a, b in ev) / 1e3
    assert int(shared["status"].item()) == 0 and tier == min(t for t in ROW_TIERS if t >= T)
    out["tier_graphs"] = dict(ms_per_step=1000.0 * sec / args.steps, value=N * args.steps / sec, tier=tier,
                              packed_rows=T, tiers=ROW_TIERS,
                              note="schedule+pack graph, read-back of the tier, then that tier's verify graph")
    return out


def bench_static(args, c, dev, drf, x):
    """The static run of the scheduled verify's data: every window the full block (no
    scheduler), 256 x 17 target rows + 256 x 16 draft rows of V = 151,936 bf16."""
    import numpy as np
    import torch
    import block_drafting_verification_amd as dsp
    R, K, V = c["R"], c["K"], c["V"]
    tgt = _bf16(dev, c["t"].reshape(R * (K + 1), V))
    cu = torch.arange(R + 1, dtype=torch.int32, device=dev) * (K + 1)
    rq = torch.arange(R, dtype=torch.int32, device=dev).repeat_interleave(K + 1)
    rp = torch.arange(K + 1, dtype=torch.int32, device=dev).repeat(R)
    rnd = torch.zeros(1, dtype=torch.int64, device=dev)
    ops = {}

    def make_step(stream):
        ver = dsp.verify_rejection(tgt, cu, x, drf=drf, temperature=1.0, seed=0, round_dev=rnd, row_req=rq,
                                   row_pos=rp, want_probs=False, stream=stream, prepare=True)
        ops["ver"] = ver
        return ver

    ph = run_phases(make_step, args.steps, args.warmup, ["VERIFY_STATS"], not args.no_flush)
    elapsed, timing = timing_record(ph, args.steps)
    assert int(ops["ver"].outputs["status"].item()) == 0, "device status flagged a fault"
    acc = ops["ver"].outputs["accepted_len"].cpu().numpy()
    N = R * K
    rows = R * (K + 1) + N
    del tgt
    return dict(workload="static run of the same data: 256 requests x 16 full windows (8,448 rows, 2.567 GB)",
                value=N * args.steps / elapsed, unit="verified draft tokens/s", ms_per_step=1000.0 * elapsed / args.steps,
                mean_accepted=float(acc.mean()),
                roofline=hbm_roofline("verify_stats", rows * V * 2, ph["kernels"]["VERIFY_STATS"]["avg_us"],
                                      traffic_from_profiles("verify.hip", "verify_stats", "scheduled-verify-static")),
                kernels=ph["kernels"], timing=timing)


# ---------------------------------------------------------------- Markov chain
def markov_cpu(c, args):
    import numpy as np
    import workloads
    from oracle import markov as om
    L = c["L"]
    U64 = workloads.bf16_bits_to_f32(c["U"]).astype(np.float64)
    W64 = workloads.bf16_bits_to_f32(c["W"]).astype(np.float64)

    def one(i):
        om.chain(workloads.bf16_bits_to_f32(L[i:i + 1]), U64, W64, c["anchors"][i:i + 1])
        return c["B"]
    return cpu_baseline(one, list(range(c["R"])), args.cpu_seconds, args.cpu_single_seconds,
                        "drafted tokens/s", "oracle greedy chain of whole requests (all 16 steps)")


def bench_markov(args, c, cpu):
    import torch
    import block_drafting_verification_amd as dsp

    dev = torch.device("cuda", 0)
    R, B, V, r = c["R"], c["B"], c["V"], c["rank"]
    L, U, Wt = _chain_l(dev, c["L"], args), _bf16(dev, c["U"]), _bf16(dev, c["W"].T)
    a = torch.from_numpy(c["anchors"]).to(dev)

    def make_step(stream):
        return dsp.draft_markov_step(L, U, Wt, a, stream=stream, prepare=True)

    persistent = args.chain_persistent
    dsp.set_option("chain_persistent", int(persistent))
    try:
        ph = run_phases(make_step, args.steps, args.warmup,
                        ["CHAIN_PERSIST" if persistent else "MARKOV_GEMM", "MARKOV_MERGE"], not args.no_flush)
    finally:
        dsp.set_option("chain_persistent", 0)
    elapsed, timing = timing_record(ph, args.steps)
    kern = ph["kernels"]
    call_bytes = R * B * V * 2 + R * B * r * 2 + V * r * 2
    if persistent:
        # one launch = the whole 16-step chain: every step's L rows and U rows, W once
        g = kern["CHAIN_PERSIST"]["avg_us"]
        bytes_launch, flops_launch, name = call_bytes, 2.0 * R * r * V * B, "chain_persist (all 16 steps)"
        per_call = g + kern["MARKOV_MERGE"]["avg_us"] * kern["MARKOV_MERGE"]["launches"] / kern["CHAIN_PERSIST"]["launches"]
    else:
        # one launch = one step over every request: the step's L rows, the previous tokens'
        # U rows, and W counted once per 16-step call (1/16 of it per step)
        g = kern["MARKOV_GEMM"]["avg_us"]
        bytes_launch, flops_launch, name = R * V * 2 + R * r * 2 + V * r * 2 // B, 2.0 * R * r * V, "markov_gemm"
        per_call = B * (g + kern["MARKOV_MERGE"]["avg_us"])
    roof = hbm_roofline(name, bytes_launch, g, traffic_from_profiles(
        "markov.hip", "chain_persist" if persistent else "markov_gemm", "markov-chain"))
    roof.update(mfma_tflops=flops_launch / (g * 1e-6) / 1e12,
                mfma_frac=flops_launch / (g * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                per_call_us=per_call,
                per_call_target_us_at_70pct=call_bytes / (0.7 * PEAK_HBM_GBS * 1e3))
    res = dict(
        metric="drafted tokens/sec", value=R * B * args.steps / elapsed, unit="tokens/s", n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=1000.0 * elapsed / args.steps, higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload="Markov-head greedy chain: 256 requests, 16 steps, V=151936, rank 256",
                    l_layout=args.l_layout, launch="persistent" if persistent else "per step"),
        roofline=roof, kernels=kern, timing=timing)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    return res


# ---------------------------------------------------------------- RNN head
def rnn_cpu(c, args):
    import numpy as np
    import workloads
    from oracle import rnn as orn
    f = workloads.bf16_bits_to_f32
    A, E, G = f(c["A"]).astype(np.float64), f(c["E"]).astype(np.float64), f(c["Gt"]).astype(np.float64).T
    Wo, b = f(c["Wo"]).astype(np.float64), c["bias"].astype(np.float64)

    def one(i):
        orn.rnn_chain(f(c["L"][i:i + 1]), f(c["h"][i:i + 1]), A, E, G, b, Wo, c["anchors"][i:i + 1])
        return c["B"]
    return cpu_baseline(one, list(range(c["R"])), args.cpu_seconds, args.cpu_single_seconds,
                        "drafted tokens/s", "oracle RNN-head chain of whole requests (all 16 steps)")


def bench_rnn(args, c, cpu):
    import torch
    import block_drafting_verification_amd as dsp

    dev = torch.device("cuda", 0)
    R, B, V, r, H = c["R"], c["B"], c["V"], c["rank"], c["H"]
    h, Gt, A, E = (_bf16(dev, c[k]) for k in ("h", "Gt", "A", "E"))
    L = _chain_l(dev, c["L"], args)
    Wot = _bf16(dev, c["Wo"].T)
    bias = _gpu(dev, c["bias"])
    a = torch.from_numpy(c["anchors"]).to(dev)

    def make_step(stream):
        return dsp.draft_rnn_step(L, h, Gt, A, E, Wot, a, bias=bias, stream=stream, prepare=True)

    ph = run_phases(make_step, args.steps, args.warmup, ["MARKOV_GEMM", "RNN_MEMO", "RNN_PROJ"], not args.no_flush)
    elapsed, timing = timing_record(ph, args.steps)
    kern = ph["kernels"]
    g = kern["MARKOV_GEMM"]["avg_us"]
    bytes_launch = R * V * 2 + R * r * 2 + V * r * 2 // B
    roof = hbm_roofline("markov_gemm (memo rows as factor rows)", bytes_launch, g, None)
    pj = kern["RNN_PROJ"]["avg_us"]
    roof["state_projection"] = dict(kernel="rnn_proj", avg_us=pj, fp64_tflops=2.0 * R * B * H * r / (pj * 1e-6) / 1e12,
                                    fp64_peak_tflops=78.6)
    res = dict(
        metric="drafted tokens/sec", value=R * B * args.steps / elapsed, unit="tokens/s", n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=1000.0 * elapsed / args.steps, higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="bf16 (projection), f64 (memo)", data="synthetic",
        config=dict(workload="RNN-head greedy chain: 256 requests, 16 steps, V=151936, rank 256, hidden 4096",
                    l_layout=args.l_layout),
        roofline=roof, kernels=kern, timing=timing)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    return res


# ---------------------------------------------------------------- PCTree
def tree_cpu(c, args):
    import numpy as np
    import workloads
    from oracle import pctree as opt
    U64 = workloads.bf16_bits_to_f32(c["U"]).astype(np.float64)
    W64 = workloads.bf16_bits_to_f32(c["W"]).astype(np.float64)

    def one(i):
        opt.tree_expand(workloads.bf16_bits_to_f32(c["L"][i:i + 1]), U64, W64, c["anchors"][i:i + 1],
                        c["topk"], c["frontier"], c["topN"])
        return c["topN"]
    return cpu_baseline(one, list(range(c["R"])), args.cpu_seconds, args.cpu_single_seconds,
                        "tree nodes/s", "oracle PCTree expansion of whole requests (16 depths)")


def bench_tree(args, c, cpu):
    import numpy as np
    import torch
    import block_drafting_verification_amd as dsp

    dev = torch.device("cuda", 0)
    R, D, V, r = c["R"], c["B"], c["V"], c["rank"]
    k, F, N = c["topk"], c["frontier"], c["topN"]
    L, U, Wt = _bf16(dev, c["L"]), _bf16(dev, c["U"]), _bf16(dev, c["W"].T)
    a = torch.from_numpy(c["anchors"]).to(dev)
    tgt = _bf16(dev, c["target"].reshape(R * (N + 1), V))
    cu = torch.arange(R + 1, dtype=torch.int32, device=dev) * (N + 1)
    ops = {}

    def make_step(stream):
        te = dsp.tree_expand(L, U, Wt, a, k, F, N, stream=stream, prepare=True)
        tv = dsp.verify_rejection(tgt, cu, te.outputs["node_token"], parent=te.outputs["node_parent"],
                                  temperature=0.0, want_probs=False, stream=stream, prepare=True)
        ops.update(te=te, tv=tv)

        def step():
            te()
            tv()
        return step

    ph = run_phases(make_step, args.steps, args.warmup, ["TREE_GEMM", "VERIFY_DECIDE"], not args.no_flush)
    elapsed, timing = timing_record(ph, args.steps)
    kern = ph["kernels"]
    f, prev = [], 1
    for _ in range(D):
        prev = min(F, k * prev)
        f.append(prev)
    parents = R * (1 + sum(f[:-1]))
    flops = 2.0 * parents * r * V
    g = kern["TREE_GEMM"]
    gemm_total_us = g["avg_us"] * g["launches"] / args.steps
    acc = ops["tv"].outputs["accepted_len"].cpu().numpy()
    walked = int((acc + 1).sum())
    tflops = flops / (gemm_total_us * 1e-6) / 1e12
    res = dict(
        metric="tree nodes/sec", value=R * N * args.steps / elapsed, unit="nodes/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=1000.0 * elapsed / args.steps, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload="PCTree expansion + greedy tree verify: 128 requests, depth 16, V=129280, rank 256, "
                             "k=4, F=16, N=64", parent_rows=parents),
        roofline=dict(kernel="tree_gemm (all depths)", bound="mfma", achieved=tflops, peak=PEAK_BF16_TFLOPS,
                      unit="TFLOP/s", frac=tflops / PEAK_BF16_TFLOPS,
                      traffic=traffic_from_profiles("markov.hip", "tree_gemm", "pctree"),
                      gemm_us_per_step=gemm_total_us, flops_per_step=flops),
        kernels=kern, timing=timing)
    # the walk reads the target rows of the visited nodes only (accepted + 1 per request)
    wk = kern["VERIFY_DECIDE"]["avg_us"]
    res["tree_verify"] = dict(kernel="verify_tree_walk", avg_us=wk, rows_walked=walked, bytes_walked=walked * V * 2,
                              GBps_walked=walked * V * 2 / (wk * 1e-6) / 1e9,
                              note="one workgroup per request walks root to leaf; latency-bound")
    if cpu is not None:
        res["cpu_baseline"] = cpu
    return res


# ---------------------------------------------------------------- closed cycle
def cycle_data():
    import numpy as np
    import workloads
    from oracle import schedule as osch
    c = workloads.cycle_case(256, 16, workloads.V_QWEN3, 256, seed=1006)
    c["w0"] = osch.schedule_windows(c["conf"], c["cost"])["windows"].astype(np.int64)
    c["tp"] = workloads.cycle_target(c, c["w0"])
    return c


def cycle_cpu(c, args):
    import numpy as np
    import workloads
    from oracle import markov as om
    from oracle import verify as ov
    U64 = workloads.bf16_bits_to_f32(c["U"]).astype(np.float64)
    W64 = workloads.bf16_bits_to_f32(c["W"]).astype(np.float64)
    cu = np.concatenate([[0], np.cumsum(c["w0"] + 1)])

    def one(i):
        d = om.chain_sampled(workloads.bf16_bits_to_f32(c["L"][i:i + 1]), U64, W64, c["anchors"][i:i + 1], 1.0,
                             seed=0, rnd=0, req_id=[i])
        n = int(c["w0"][i])
        t = workloads.bf16_bits_to_f32(c["tp"][cu[i]:cu[i + 1]])
        ov.verify_chain(t, np.array([0, n + 1]), d["zhat"], d["y"], 1.0, seed=0, rnd=1, req_id=[i])
        return n
    return cpu_baseline(one, list(range(c["R"])), args.cpu_seconds, args.cpu_single_seconds,
                        "verified draft tokens/s",
                        "oracle sampled draft (16 steps) + verify of whole requests (the scheduler's windows)")


def bench_cycle(args, c, cpu):
    """Draft -> confidence head -> schedule -> pack -> verify, one HIP graph per step (the
    pages' cycle). The Markov head samples 16 positions for 256 requests and emits its bf16
    rows (the verify's q); the confidence head (hidden size 4096, sequential temperatures)
    gives the per-position confidences from which the scheduler picks windows; the pack lays
    out the verify buffer; the verify checks the windows against target rows laid out in
    packed order at setup (they stand in for the target forward, which is not part of the
    method and is not timed)."""
    import numpy as np
    import torch
    import block_drafting_verification_amd as dsp
    import workloads

    dev = torch.device("cuda", 0)
    R, K, V, r = c["R"], c["K"], c["V"], c["rank"]
    L, U, Wt = _chain_l(dev, c["L"], args), _bf16(dev, c["U"]), _bf16(dev, c["W"].T)
    a = torch.from_numpy(c["anchors"]).to(dev)
    hd = workloads.cycle_head_inputs(c)
    hh, hw = _bf16(dev, hd["h"]), _bf16(dev, hd["w"])
    temps = torch.from_numpy(hd["temps"]).to(dev)
    cost = torch.from_numpy(c["cost"]).to(dev)
    conf0 = dsp.confidence_head(hh, hw, hd["bias"], temps)["conf"]
    w0 = dsp.schedule_windows(conf0, cost)["windows"].cpu().numpy()
    assert np.array_equal(w0, c["w0"]), "the head's confidences give other windows than the workload's"
    # packed target rows at the front of a buffer for the largest batch (the step is captured
    # once with max_rows = R x (K+1); its kernels skip the rows past the device-side total)
    tgt = torch.zeros(R * (K + 1), V, dtype=torch.bfloat16, device=dev)
    tgt[:c["tp"].shape[0]].copy_(_bf16(dev, c["tp"]))
    rd = torch.zeros(1, dtype=torch.int64, device=dev)
    ops = {}

    def make_step(stream):
        dr = dsp.draft_markov_sample(L, U, Wt, a, 1.0, seed=0, round_dev=rd, stream=stream, prepare=True)
        ch = dsp.confidence_head(hh, hw, hd["bias"], temps, stream=stream, prepare=True)
        sch = dsp.schedule_pack(ch.outputs["conf"], cost, a, dr.outputs["y"], want_survival=False, stream=stream,
                                prepare=True)
        ver = dsp.verify_rejection(tgt, sch.outputs["cu_seqlens"], dr.outputs["y"], drf=dr.outputs["z"],
                                   temperature=1.0, seed=0, round_dev=rd, max_rows=tgt.shape[0],
                                   row_req=sch.outputs["row_req"], row_pos=sch.outputs["row_pos"],
                                   want_probs=False, stream=stream, prepare=True)
        ops.update(dr=dr, ch=ch, sch=sch, ver=ver)

        def step():
            dr()
            ch()
            sch()
            ver()
        return step

    ph = run_phases(make_step, args.steps, args.warmup, ["MARKOV_GEMM", "VERIFY_STATS"], not args.no_flush)
    elapsed, timing = timing_record(ph, args.steps)
    kern = ph["kernels"]
    for k in ("dr", "ch", "sch", "ver"):
        assert int(ops[k].outputs["status"].item()) == 0, "device status flagged a fault"
    win = ops["sch"].outputs["windows"].cpu().numpy()
    assert np.array_equal(win, w0)
    N = int(win.sum())
    acc = ops["ver"].outputs["accepted_len"].cpu().numpy()
    g = kern["MARKOV_GEMM"]["avg_us"]
    # one sampled step: L rows, previous tokens' U rows, W once per 16-step call, emitted rows
    bytes_launch = R * V * 2 + R * r * 2 + V * r * 2 // K + R * V * 2
    res = dict(
        metric="verified draft tokens/sec", value=N * args.steps / elapsed, unit="tokens/s", n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=1000.0 * elapsed / args.steps, higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="bf16",
        data="synthetic (Markov-head inputs; target rows = draft base logits + per-request noise, packed order)",
        config=dict(workload="draft -> confidence head -> schedule -> pack -> verify cycle: 256 requests, "
                             "16 sampled drafts, V=151936, rank 256, hidden 4096, T=1, additive cost 1+0.05n",
                    requests=R, block=K, vocab=V, drafted_per_step=R * K, verified_drafts_per_step=N,
                    packed_rows=R + N, mean_accepted=float(acc.mean()), l_layout=args.l_layout,
                    drafted_tokens_per_s=R * K * args.steps / elapsed),
        roofline=hbm_roofline("markov_gemm (sampled, emits bf16 rows)", bytes_launch, g,
                              traffic_from_profiles("markov.hip", "markov_gemm", "cycle")),
        kernels=kern, timing=timing)
    if cpu is not None:
        res["cpu_baseline"] = cpu
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
    want_cpu = not args.no_cpu_baseline
    # host side first (data, then the CPU oracle sample), before anything touches the GPU
    w = args.workload
    if w in ("dense-verify", "scheduled-verify"):
        c = verify_data(w)
        cpu = verify_cpu(c, args) if want_cpu else None
    elif w == "markov-chain":
        import workloads
        c = workloads.markov_chain()
        cpu = markov_cpu(c, args) if want_cpu else None
    elif w == "rnn-chain":
        import workloads
        c = workloads.rnn_case(256, 16, workloads.V_QWEN3, 256, H=4096, seed=1007)
        cpu = rnn_cpu(c, args) if want_cpu else None
    elif w == "pctree":
        import workloads
        c = workloads.pctree()
        cpu = tree_cpu(c, args) if want_cpu else None
    elif w == "cycle":
        c = cycle_data()
        cpu = cycle_cpu(c, args) if want_cpu else None
    import torch
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.general_gemm:
        import block_drafting_verification_amd as dsp
        dsp.set_option("chain_sched", 0)
        dsp.set_option("tree_split", 0)
    if w == "copy":
        res = bench_copy(args)
    elif w in ("dense-verify", "scheduled-verify"):
        res = bench_verify(args, w, c, cpu)
    elif w == "markov-chain":
        res = bench_markov(args, c, cpu)
    elif w == "rnn-chain":
        res = bench_rnn(args, c, cpu)
    elif w == "cycle":
        res = bench_cycle(args, c, cpu)
    else:
        res = bench_tree(args, c, cpu)
    if args.general_gemm:
        res["config"]["gemm"] = "general (diagnostic)"
    print(json.dumps(res))


if __name__ == "__main__":
    main()
