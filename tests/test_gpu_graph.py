"""HIP-graph replay of whole steps against eager execution of the same prepared calls.

The timed steps replay one captured graph per step. A replay must give, bit for bit,
what the same calls give when issued eagerly for the same round: the device round
counter is the only state that moves between steps (the verify advances it), and
every workspace a kernel reads is written by an earlier kernel of the same step.
Each test runs a few steps eagerly, captures the step once, resets the round and
replays it, with unrelated eager work and synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

import block_drafting_verification_amd as dsp
import workloads
from parity import logits_to_gpu, packed_from_dense, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

STEPS = 3


def _snapshot(ops, keys):
    return {f"{o}.{k}": ops[o].outputs[k].clone() for o, k in keys}


def _unrelated_eager_work(dev):
    a = torch.randn(512, 512, device=dev)
    _ = (a @ a).sum().item()
    conf = torch.rand(8, 4, device=dev, dtype=torch.float32)
    cost = torch.arange(33, device=dev, dtype=torch.float64) * 0.05 + 1.0
    dsp.schedule_windows(conf, cost)
    torch.cuda.synchronize()


def _replay_matches_eager(make_step, ops, keys, rd, dev):
    s = torch.cuda.Stream()
    step = make_step(s)
    eager = []
    with torch.cuda.stream(s):
        rd.zero_()
    for _ in range(STEPS):
        step()
        torch.cuda.synchronize()
        eager.append(_snapshot(ops, keys))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    with torch.cuda.stream(s):
        rd.zero_()
    torch.cuda.synchronize()
    for r in range(STEPS):
        print(f"graph replay {r}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(ops, keys)
        for name, ref in eager[r].items():
            assert torch.equal(got[name], ref), (r, name)
        _unrelated_eager_work(dev)
    assert int(rd.item()) == STEPS
    # the steps drew fresh uniforms: the drafts of two rounds differ
    first = [n for n in eager[0] if n.endswith(".y")]
    assert all(not torch.equal(eager[0][n], eager[1][n]) for n in first)


def test_graph_cycle_replays_match_eager():
    """Sampled draft -> confidence head -> schedule -> pack -> verify, 256 requests x 16,
    V=30,011."""
    dev = torch.device("cuda", 0)
    c = workloads.cycle_case(256, 16, 30011, 64, seed=2024)
    L, U = to_gpu_bf16(c["L"]), to_gpu_bf16(c["U"])
    Wt = to_gpu_bf16(np.ascontiguousarray(c["W"].T))
    a = to_gpu(c["anchors"].astype(np.int32))
    hd = workloads.cycle_head_inputs(c, H=512)
    hh, hw = to_gpu_bf16(hd["h"]), to_gpu_bf16(hd["w"])
    temps = to_gpu(hd["temps"])
    cost = to_gpu(c["cost"])
    conf0 = dsp.confidence_head(hh, hw, hd["bias"], temps)["conf"]
    w0 = dsp.schedule_windows(conf0, cost)["windows"].cpu().numpy()
    tgt = to_gpu_bf16(workloads.cycle_target(c, w0))
    rd = torch.zeros(1, dtype=torch.int64, device=dev)
    ops = {}
    print(f"graph cycle R=256 K=16 V=30011 packed rows={tgt.shape[0]}", flush=True)

    def make_step(stream):
        dr = dsp.draft_markov_sample(L, U, Wt, a, 1.0, seed=7, round_dev=rd, stream=stream, prepare=True)
        ch = dsp.confidence_head(hh, hw, hd["bias"], temps, stream=stream, prepare=True)
        sch = dsp.schedule_windows(ch.outputs["conf"], cost, stream=stream, prepare=True)
        pk = dsp.pack_ragged(sch.outputs["windows"], a, dr.outputs["y"], stream=stream, prepare=True)
        ver = dsp.verify_rejection(tgt, pk.outputs["cu_seqlens"], dr.outputs["y"], drf=dr.outputs["z"],
                                   temperature=1.0, seed=7, round_dev=rd, max_rows=tgt.shape[0],
                                   row_req=pk.outputs["row_req"], row_pos=pk.outputs["row_pos"],
                                   stream=stream, prepare=True)
        ops.update(dr=dr, ch=ch, sch=sch, pk=pk, ver=ver)

        def step():
            dr()
            ch()
            sch()
            pk()
            ver()
        return step

    keys = [("dr", "y"), ("dr", "z"), ("dr", "logq"), ("ch", "conf"), ("sch", "windows"),
            ("sch", "survival"), ("pk", "cu_seqlens"), ("pk", "tokens"), ("ver", "accepted_len"),
            ("ver", "out_tokens"), ("ver", "p_x"), ("ver", "q_x")]
    _replay_matches_eager(make_step, ops, keys, rd, dev)
    for k in ("dr", "ch", "pk", "ver"):
        assert int(ops[k].outputs["status"].item()) == 0


def test_graph_dense_verify_replays_match_eager():
    """Schedule + pack (one call) -> verify, 64 requests x K=7 (decision, residual and draw as
    three launches), V=40,000, with the round on the device."""
    dev = torch.device("cuda", 0)
    c = workloads.verify_case(64, 7, 40000, dtype="bf16", seed=31, boost_p=0.01)
    R, K = c["R"], c["K"]
    conf = to_gpu(np.full((R, K), 0.99, dtype=np.float32))
    cost = to_gpu(np.ones(R * K + 1))
    tp = packed_from_dense(c["t"], np.full(R, K))
    tgt = logits_to_gpu(tp, "bf16")
    drf = logits_to_gpu(c["d"], "bf16")
    x = to_gpu(c["x"].astype(np.int32))
    anchors = to_gpu(np.arange(R, dtype=np.int32))
    rd = torch.zeros(1, dtype=torch.int64, device=dev)
    ops = {}

    def make_step(stream):  # the scheduler and the pack in one call, as the bench runs them
        sch = dsp.schedule_pack(conf, cost, anchors, x, stream=stream, prepare=True)
        pk = sch
        ver = dsp.verify_rejection(tgt, pk.outputs["cu_seqlens"], x, drf=drf, temperature=1.0, seed=3,
                                   round_dev=rd, max_rows=tgt.shape[0], row_req=pk.outputs["row_req"],
                                   row_pos=pk.outputs["row_pos"], stream=stream, prepare=True)
        ops.update(sch=sch, pk=pk, ver=ver)

        def step():
            sch()
            ver()
        return step

    keys = [("sch", "windows"), ("pk", "cu_seqlens"), ("ver", "accepted_len"), ("ver", "out_tokens"),
            ("ver", "p_x"), ("ver", "q_x")]
    s = torch.cuda.Stream()
    step = make_step(s)
    eager = []
    for _ in range(STEPS):
        step()
        torch.cuda.synchronize()
        eager.append(_snapshot(ops, keys))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    with torch.cuda.stream(s):
        rd.zero_()
    torch.cuda.synchronize()
    for r in range(STEPS):
        print(f"graph replay {r}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(ops, keys)
        for name, ref in eager[r].items():
            assert torch.equal(got[name], ref), (r, name)
        _unrelated_eager_work(dev)
    assert int(rd.item()) == STEPS
    assert not torch.equal(eager[0]["ver.out_tokens"], eager[1]["ver.out_tokens"])
    assert int(ops["ver"].outputs["status"].item()) == 0


def test_graph_tree_expand_replays_match_eager():
    """PCTree expansion (probe pass, row bounds, per-depth GEMM and merge) as one graph."""
    dev = torch.device("cuda", 0)
    c = workloads.markov_case(16, 6, 20011, rank=64, seed=77)
    L, U = to_gpu_bf16(c["L"]), to_gpu_bf16(c["U"])
    Wt = to_gpu_bf16(np.ascontiguousarray(c["W"].T))
    a = to_gpu(c["anchors"].astype(np.int32))
    s = torch.cuda.Stream()
    t = dsp.tree_expand(L, U, Wt, a, 4, 16, 40, want_mask=True, stream=s, prepare=True)
    keys = ["node_token", "node_parent", "node_depth", "node_score", "n_nodes", "anc_mask"]
    t()
    torch.cuda.synchronize()
    ref = {k: t.outputs[k].clone() for k in keys}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        t()
    for r in range(STEPS):
        for k in keys:  # scribble over the outputs: a replay must rewrite them
            t.outputs[k].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(t.outputs[k], ref[k]), (r, k)
        _unrelated_eager_work(dev)
    assert int(t.outputs["status"].item()) == 0


def test_tier_graph_replays_match_eager():
    """Per-tier graph replay (SGLang article, "Ragged verify"): one verify graph captured per
    packed-row tier, chosen each step by the tier the pack wrote; every step's outputs
    equal an eager verify of the same packing over the full row range, bit for bit.
    48 requests x K=8, V=20,000, windows moving from short to long across the steps."""
    dev = torch.device("cuda", 0)
    R, K, V = 48, 8, 20000
    c = workloads.verify_case(R, K, V, dtype="bf16", seed=77, boost_p=0.01, d_sigma=0.8)
    rng = np.random.default_rng(78)
    tiers = [64, 96, 160, 288, R * (K + 1)]
    drf = logits_to_gpu(c["d"], "bf16")
    x = to_gpu(c["x"].astype(np.int32))
    anchors = to_gpu(np.arange(R, dtype=np.int32))
    cost = to_gpu(1.0 + 0.05 * np.arange(R * K + 1))
    conf = torch.zeros(R, K, dtype=torch.float32, device=dev)
    tgt = torch.zeros(R * (K + 1), V, dtype=torch.bfloat16, device=dev)
    rd = torch.zeros(1, dtype=torch.int64, device=dev)
    rd_ref = torch.zeros(1, dtype=torch.int64, device=dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        sch = dsp.schedule_pack(conf, cost, anchors, x, tiers=tiers, stream=s, prepare=True)
    shared = {"status": torch.zeros(1, dtype=torch.int32, device=dev)}

    def make(tier):  # every tier's call writes the same output buffers
        v = dsp.verify_rejection(tgt, sch.outputs["cu_seqlens"], x, drf=drf, temperature=1.0, seed=5,
                                 round_dev=rd, max_rows=tier, row_req=sch.outputs["row_req"],
                                 row_pos=sch.outputs["row_pos"], out=shared, status=shared["status"],
                                 stream=s, prepare=True)
        shared.update({k: t for k, t in v.outputs.items() if t is not None})
        return v

    tg = dsp.TierGraphs(tiers, make, stream=s)
    used = set()
    for step, mu in enumerate([-1.5, 0.5, 2.5, 5.0, 0.0]):
        c_s = (1.0 / (1.0 + np.exp(-(mu + rng.standard_normal((R, K)))))).astype(np.float32)
        conf.copy_(to_gpu(c_s))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            sch()
        s.synchronize()
        win = sch.outputs["windows"].cpu().numpy()
        T = int(win.sum()) + R
        tgt[:T].copy_(logits_to_gpu(packed_from_dense(c["t"], win), "bf16"))
        torch.cuda.synchronize()
        print(f"tier step {step}: packed rows {T}", flush=True)
        tier = tg.replay(sch.outputs["total_and_tier"])
        assert tier == min(t for t in tiers if t >= T)
        assert sch.outputs["total_and_tier"].cpu().tolist() == [T, tier]
        used.add(tier)
        s.synchronize()
        got = {k: shared[k].clone() for k in ("accepted_len", "out_tokens", "stop_pos", "p_x", "q_x", "status")}
        ref = dsp.verify_rejection(tgt, sch.outputs["cu_seqlens"], x, drf=drf, temperature=1.0, seed=5,
                                   round_dev=rd_ref, row_req=sch.outputs["row_req"], row_pos=sch.outputs["row_pos"])
        torch.cuda.synchronize()
        for k, t in got.items():
            assert torch.equal(t, ref[k]), (step, k)
        assert int(got["status"].item()) == 0
        _unrelated_eager_work(dev)
    assert len(used) >= 3, used
    assert int(rd.item()) == int(rd_ref.item()) == 5
