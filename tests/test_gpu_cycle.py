"""GPU parity of the full draft -> schedule -> pack -> verify cycle against the oracle.

The cycle of the DSpark study notes (sections 1, 4, 5) as the SGLang article runs
it ("Ragged verify"): the Markov head drafts K positions per request by sampling
and emits its bf16 logit rows; the scheduler turns per-position confidences into
windows; the pack lays the anchors and windowed drafts out front to back; the
verify checks the drafts against the target rows of the packed buffer, with the
draft's own emitted rows as q. The target forward is not part of the method: its
output rows are synthetic, laid out in packed order. One device round counter is
shared: the draft reads it, the verify advances it and uses the new value.
"""
import numpy as np
import pytest
import torch

import block_drafting_verification_amd as dsp
import workloads
from oracle import markov as om
from oracle import pack as opack
from oracle import schedule as osch
from oracle import verify as ov
from parity import SAMPLE_BAND, TieCounter, compare_chain_verify, host, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _run_cycle(c, T, seed):
    R, K, V = c["R"], c["K"], c["V"]
    L, U, W = (workloads.bf16_bits_to_f32(c[k]) for k in ("L", "U", "W"))
    windows_host = osch.schedule_windows(c["conf"], c["cost"])["windows"]
    tp = workloads.cycle_target(c, windows_host)
    print(f"cycle R={R} K={K} V={V} rank={c['rank']} T={T} packed rows={tp.shape[0]}", flush=True)
    Lg, Ug = to_gpu_bf16(c["L"]), to_gpu_bf16(c["U"])
    Wtg = to_gpu_bf16(np.ascontiguousarray(c["W"].T))
    ag = to_gpu(c["anchors"].astype(np.int32))
    rd = torch.zeros(1, dtype=torch.int64, device=Lg.device)
    dr = dsp.draft_markov_sample(Lg, Ug, Wtg, ag, T, seed=seed, round_dev=rd)
    sch = dsp.schedule_windows(to_gpu(c["conf"]), to_gpu(c["cost"]))
    pk = dsp.pack_ragged(sch["windows"], ag, dr["y"])
    ver = dsp.verify_rejection(to_gpu_bf16(tp), pk["cu_seqlens"], dr["y"], drf=dr["z"], temperature=T,
                               seed=seed, round_dev=rd, row_req=pk["row_req"], row_pos=pk["row_pos"],
                               want_probs=False)
    torch.cuda.synchronize()
    for st in (dr["status"], pk["status"], ver["status"]):
        assert int(host(st)[0]) == 0
    assert int(host(rd)[0]) == 1

    # draft: the oracle replays the GPU's draws (each step checked locally)
    y = host(dr["y"]).astype(np.int64)
    od = om.chain_sampled(L, U, W, c["anchors"], T, seed=seed, rnd=0, forced=y)
    ties = TieCounter()
    ties.decisions += y.size
    for i, d in np.argwhere(od["y"] != y):
        assert od["sample_margin"][i, d] < SAMPLE_BAND + od["tie_shift"][i, d], (i, d)
        ties.near += 1
    # schedule and pack: exact
    w = host(sch["windows"])
    np.testing.assert_array_equal(w, windows_host)
    op = opack.pack_ragged(w, c["anchors"], y)
    np.testing.assert_array_equal(host(pk["cu_seqlens"]), op["cu_seqlens"])
    T_rows = int(op["cu_seqlens"][-1])
    np.testing.assert_array_equal(host(pk["tokens"])[:T_rows], op["tokens"])
    # verify, q = the oracle's own rounded draft rows; where a draft row has rounding
    # near-ties the two sides' q may differ slightly, and the bands widen by that row's bound
    tv = workloads.bf16_bits_to_f32(tp).astype(np.float64)

    def orc(forced):
        return ov.verify_chain(tv, op["cu_seqlens"], od["zhat"], y, T, seed=seed, rnd=1, forced_len=forced)
    compare_chain_verify(ver, orc, R, K, w, ties, draft_bounds=(od["eps"], od["tok_dev"], T))
    ties.check()
    acc = host(ver["accepted_len"])
    return w, acc


@pytest.mark.parametrize("R,K,V,rank,T", [(8, 5, 2003, 32, 1.0), (40, 7, 9001, 64, 0.8), (6, 16, 30011, 256, 1.0)])
def test_cycle_small(R, K, V, rank, T):
    c = workloads.cycle_case(R, K, V, rank, seed=R * 31 + V)
    w, acc = _run_cycle(c, T, seed=5)
    assert w.sum() > 0
    assert np.all(acc <= w)


def test_cycle_repeats_draw_fresh_uniforms():
    """Two cycles on one device round counter: the second draws with round 1 (draft) and 2 (verify)."""
    c = workloads.cycle_case(8, 5, 2003, 32, seed=77)
    Lg, Ug = to_gpu_bf16(c["L"]), to_gpu_bf16(c["U"])
    Wtg = to_gpu_bf16(np.ascontiguousarray(c["W"].T))
    ag = to_gpu(c["anchors"].astype(np.int32))
    rd = torch.zeros(1, dtype=torch.int64, device=Lg.device)
    ys = []
    for _ in range(2):
        dr = dsp.draft_markov_sample(Lg, Ug, Wtg, ag, 1.0, seed=3, round_dev=rd)
        rd += 1  # stands in for the verify's advance
        ys.append(host(dr["y"]))
    torch.cuda.synchronize()
    L, U, W = (workloads.bf16_bits_to_f32(c[k]) for k in ("L", "U", "W"))
    for rnd, y in enumerate(ys):
        o = om.chain_sampled(L, U, W, c["anchors"], 1.0, seed=3, rnd=rnd, forced=y.astype(np.int64))
        bad = np.argwhere(o["y"] != y)
        assert all(o["sample_margin"][i, d] < SAMPLE_BAND + o["tie_shift"][i, d] for i, d in bad)
    assert not np.array_equal(ys[0], ys[1])


def test_cycle_bench_shape_sampled_requests():
    """The cycle at the bench's shape (256 requests x 16 sampled drafts, V=151,936, rank 256):
    windows and pack checked exactly for every request; draws (all 16 steps, replayed) and the
    verify decisions and drawn tokens checked against the oracle on sampled requests."""
    c = workloads.cycle_case(256, 16, workloads.V_QWEN3, 256, seed=1006)
    R, K, V, T, seed = c["R"], c["K"], c["V"], 1.0, 0
    L, U, W = (workloads.bf16_bits_to_f32(c[k]) for k in ("L", "U", "W"))
    windows_host = osch.schedule_windows(c["conf"], c["cost"])["windows"]
    tp = workloads.cycle_target(c, windows_host)
    print(f"cycle (bench shape) packed rows={tp.shape[0]} drafts={int(windows_host.sum())}", flush=True)
    Lg, Ug = to_gpu_bf16(c["L"]), to_gpu_bf16(c["U"])
    Wtg = to_gpu_bf16(np.ascontiguousarray(c["W"].T))
    ag = to_gpu(c["anchors"].astype(np.int32))
    rd = torch.zeros(1, dtype=torch.int64, device=Lg.device)
    dr = dsp.draft_markov_sample(Lg, Ug, Wtg, ag, T, seed=seed, round_dev=rd)
    sch = dsp.schedule_windows(to_gpu(c["conf"]), to_gpu(c["cost"]))
    pk = dsp.pack_ragged(sch["windows"], ag, dr["y"])
    ver = dsp.verify_rejection(to_gpu_bf16(tp), pk["cu_seqlens"], dr["y"], drf=dr["z"], temperature=T,
                               seed=seed, round_dev=rd, row_req=pk["row_req"], row_pos=pk["row_pos"],
                               want_probs=False)
    torch.cuda.synchronize()
    for st in (dr["status"], pk["status"], ver["status"]):
        assert int(host(st)[0]) == 0
    y = host(dr["y"]).astype(np.int64)
    w = host(sch["windows"])
    np.testing.assert_array_equal(w, windows_host)
    op = opack.pack_ragged(w, c["anchors"], y)
    np.testing.assert_array_equal(host(pk["cu_seqlens"]), op["cu_seqlens"])
    T_rows = int(op["cu_seqlens"][-1])
    np.testing.assert_array_equal(host(pk["tokens"])[:T_rows], op["tokens"])
    sel = np.array([0, 5, 77, 128, 200, 255])
    od = om.chain_sampled(L[sel], U, W, c["anchors"][sel], T, seed=seed, rnd=0, req_id=sel, forced=y[sel])
    ties = TieCounter()
    ties.decisions += y[sel].size
    for ii, d in np.argwhere(od["y"] != y[sel]):
        assert od["sample_margin"][ii, d] < SAMPLE_BAND + od["tie_shift"][ii, d], (sel[ii], d)
        ties.near += 1
    # verify of the sampled requests: their packed rows and their own draft rows as q
    cu = op["cu_seqlens"]
    rows = np.concatenate([tp[cu[i]:cu[i + 1]] for i in sel])
    cu_s = np.concatenate([[0], np.cumsum([cu[i + 1] - cu[i] for i in sel])]).astype(np.int32)
    tv = workloads.bf16_bits_to_f32(rows).astype(np.float64)

    def orc(forced):
        return ov.verify_chain(tv, cu_s, od["zhat"], y[sel], T, seed=seed, rnd=1, req_id=sel, forced_len=forced)
    sub = {k: ver[k][torch.as_tensor(sel, device=ver[k].device)] for k in ("accepted_len", "out_tokens")}
    compare_chain_verify(sub, orc, len(sel), K, w[sel], ties, draft_bounds=(od["eps"], od["tok_dev"], T))
    ties.check()
