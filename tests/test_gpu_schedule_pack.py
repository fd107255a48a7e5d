"""GPU parity of the confidence scheduler and the ragged pack (bit-exact against the oracle)."""
import numpy as np
import pytest
import torch

import block_drafting_verification_amd as dsp
import workloads
from oracle import pack as opack
from oracle import schedule as osch
from parity import host, to_gpu

pytestmark = pytest.mark.gpu


def _sched(conf, cost, mode=0, cap=-1, threshold=0.0):
    print(f"schedule R={conf.shape[0]} K={conf.shape[1]} mode={mode} cap={cap} th={threshold}", flush=True)
    g = dsp.schedule_windows(to_gpu(conf), to_gpu(cost), mode=mode, max_tokens=cap, threshold=threshold)
    torch.cuda.synchronize()
    o = osch.schedule_windows(conf, cost, mode=mode, max_tokens=cap, threshold=threshold)
    np.testing.assert_array_equal(host(g["windows"]), o["windows"])
    np.testing.assert_array_equal(host(g["survival"]), o["survival"])
    st = host(g["stats"])
    assert st[0] == o["N"] and st[1] == o["E"] and st[3] == o["Q"]
    assert st[2] == o["J"]
    return o


@pytest.mark.parametrize("R,K", [(1, 1), (3, 2), (7, 16), (64, 7), (256, 16), (100, 33), (8192, 1), (64, 128)])
def test_schedule_random(R, K):
    rng = np.random.Generator(np.random.PCG64(R * 1000 + K))
    conf = rng.uniform(0.0, 1.0, size=(R, K)).astype(np.float32)
    conf[rng.random((R, K)) < 0.05] = 1.0
    for a, b in [(1.0, 0.05), (1.0, 0.0), (0.3, 0.2)]:
        cost = osch.additive_cost(a, b, R * K)
        for mode in (osch.MODE_EARLY_STOP, osch.MODE_ARGMAX):
            _sched(conf, cost, mode)
    _sched(conf, osch.additive_cost(1.0, 0.01, R * K), 0, cap=max(1, R * K // 3))
    # non-smooth measured table (random positive steps)
    cost = np.cumsum(rng.uniform(0.0, 0.2, size=R * K + 1)) + 1.0
    cost[rng.random(R * K + 1) < 0.1] += 0.5
    _sched(conf, cost, 0)
    _sched(conf, cost, 1)


@pytest.mark.parametrize("R,K", [(64, 16), (256, 16), (32, 128)])
def test_schedule_misaligned_inputs(R, K):
    """conf one float and cost one double past a 16-byte boundary: the ranking reads the
    confidence rows with scalar loads instead of 16-byte ones; the result is the same."""
    rng = np.random.Generator(np.random.PCG64(R * 7 + K))
    conf = rng.uniform(0.0, 1.0, size=(R, K)).astype(np.float32)
    conf[rng.random((R, K)) < 0.05] = 1.0
    cost = osch.additive_cost(1.0, 0.05, R * K)
    cbuf = torch.zeros(R * K + 1, dtype=torch.float32, device="cuda")
    cbuf[1:] = to_gpu(conf).reshape(-1)
    conf_v = cbuf[1:].view(R, K)
    kbuf = torch.zeros(cost.size + 1, dtype=torch.float64, device="cuda")
    kbuf[1:] = to_gpu(cost)
    cost_v = kbuf[1:]
    assert conf_v.data_ptr() % 16 == 4 and cost_v.data_ptr() % 16 == 8
    for mode in (osch.MODE_EARLY_STOP, osch.MODE_ARGMAX):
        print(f"schedule misaligned R={R} K={K} mode={mode}", flush=True)
        g = dsp.schedule_windows(conf_v, cost_v, mode=mode)
        torch.cuda.synchronize()
        o = osch.schedule_windows(conf, cost, mode=mode)
        np.testing.assert_array_equal(host(g["windows"]), o["windows"])
        np.testing.assert_array_equal(host(g["survival"]), o["survival"])
        st = host(g["stats"])
        assert st[0] == o["N"] and st[1] == o["E"] and st[2] == o["J"] and st[3] == o["Q"]


@pytest.mark.parametrize("R,K", [(3, 5), (64, 7), (256, 16)])
def test_schedule_nonmonotone_survival(R, K):
    """Confidences above 1 let a survival grow along k, so a request's candidates are no
    longer ranked in position order: the kernel must see it and sort every key."""
    rng = np.random.Generator(np.random.PCG64(77 + R * K))
    S = rng.uniform(0.05, 1.0, size=(R, K))
    prev = np.concatenate([np.ones((R, 1)), S[:, :-1]], axis=1)
    conf = (S / prev).astype(np.float32)
    assert np.any(conf > 1.0)
    for mode in (osch.MODE_EARLY_STOP, osch.MODE_ARGMAX):
        _sched(conf, osch.additive_cost(1.0, 0.05, R * K), mode)
    _sched(conf, osch.additive_cost(1.0, 0.05, R * K), osch.MODE_TOP_M, cap=R * K // 2)


def test_schedule_special_cases():
    R, K = 16, 8
    cost = osch.additive_cost(1.0, 0.05, R * K)
    o = _sched(np.ones((R, K), np.float32), cost)
    assert np.all(o["windows"] == K)
    o = _sched(np.zeros((R, K), np.float32), cost)
    assert np.all(o["windows"] == 0)
    o = _sched(np.zeros((R, K), np.float32), np.zeros(R * K + 1))
    assert np.all(o["windows"] == 0)


@pytest.mark.parametrize("R,K", [(256, 16), (512, 16), (8192, 1)])
def test_schedule_ties_across_requests(R, K):
    """Survivals that tie across many requests (a constant confidence; rows repeated
    request to request) at up to the largest candidate count: the order falls back to
    (request, position), so a capacity cut through a tied run must take the lower
    requests first, exactly as the oracle does."""
    rng = np.random.Generator(np.random.PCG64(R * 11 + K))
    row = rng.uniform(0.3, 1.0, size=(1, K)).astype(np.float32)
    for conf in (np.full((R, K), 0.5, np.float32), np.repeat(row, R, axis=0)):
        cost = osch.additive_cost(1.0, 0.01, R * K)
        for mode in (osch.MODE_EARLY_STOP, osch.MODE_ARGMAX):
            _sched(conf, cost, mode)
        for cap in (1, R // 3, R * K // 2 + 1):
            o = _sched(conf, cost, osch.MODE_TOP_M, cap=cap)
            assert o["windows"].sum() == cap


@pytest.mark.parametrize("R,K", [(1, 1), (7, 16), (64, 7), (256, 16), (8192, 1), (64, 128)])
def test_schedule_top_m_and_threshold(R, K):
    rng = np.random.Generator(np.random.PCG64(R * 7 + K))
    conf = rng.uniform(0.0, 1.0, size=(R, K)).astype(np.float32)
    conf[rng.random((R, K)) < 0.05] = 1.0
    cost = osch.additive_cost(1.0, 0.05, R * K)
    for M in sorted({0, 1, R * K // 5, R * K // 2, R * K}):
        _sched(conf, cost, osch.MODE_TOP_M, cap=M)
    for th in (0.0, 1e-6, 0.1, 0.5, 0.9, 1.0, 1.5):
        _sched(conf, cost, osch.MODE_THRESHOLD, threshold=th)


def test_schedule_c3_workload():
    c = workloads.scheduled_verify_schedule_inputs()
    for th in (0.3, 0.6):
        _sched(c["conf"], c["cost"], osch.MODE_THRESHOLD, threshold=th)
    o = _sched(c["conf"], c["cost"])
    _sched(c["conf"], c["cost"], osch.MODE_TOP_M, cap=o["N"])
    print("scheduled verify: N =", o["N"], "of", 256 * 16)
    assert 0 < o["N"] < 256 * 16


@pytest.mark.parametrize("R,K", [(1, 1), (5, 3), (256, 16), (4000, 7)])
def test_pack_random(R, K):
    rng = np.random.Generator(np.random.PCG64(R + K))
    w = rng.integers(0, K + 1, size=R).astype(np.int32)
    anchors = rng.integers(0, 10**6, size=R).astype(np.int32)
    drafts = rng.integers(0, 10**6, size=(R, K)).astype(np.int32)
    tiers = sorted(set(rng.integers(R, R * (K + 1) + 2, size=8).tolist()))
    print(f"pack R={R} K={K}", flush=True)
    for tl in (None, tiers):
        g = dsp.pack_ragged(to_gpu(w), to_gpu(anchors), to_gpu(drafts), tiers=tl)
        torch.cuda.synchronize()
        o = opack.pack_ragged(w, anchors, drafts, tiers=tl)
        T = o["total"]
        np.testing.assert_array_equal(host(g["cu_seqlens"]), o["cu_seqlens"])
        np.testing.assert_array_equal(host(g["tokens"])[:T], o["tokens"])
        np.testing.assert_array_equal(host(g["row_req"])[:T], o["row_req"])
        np.testing.assert_array_equal(host(g["row_pos"])[:T], o["row_pos"])
        assert host(g["total_and_tier"]).tolist() == [T, o["tier"]]
        assert int(host(g["status"])[0]) == 0


def test_pack_flags_bad_window():
    w = np.array([2, 9, 1], np.int32)
    g = dsp.pack_ragged(to_gpu(w), to_gpu(np.zeros(3, np.int32)), to_gpu(np.zeros((3, 4), np.int32)))
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) & dsp.DSP_STATUS_WINDOW_RANGE


@pytest.mark.parametrize("R,K", [(1, 1), (7, 16), (64, 7), (256, 16), (2000, 4), (64, 128), (8192, 1)])
def test_schedule_pack_one_call(R, K):
    """dsp_schedule_pack equals dsp_schedule_windows then dsp_pack_ragged, bit for bit, in every
    scheduler mode, with and without tiers; the windows and pack also against the oracle."""
    rng = np.random.Generator(np.random.PCG64(R * 7 + K))
    conf = rng.uniform(0.05, 1.0, size=(R, K)).astype(np.float32)
    cost = 1.0 + 0.05 * np.arange(R * K + 1, dtype=np.float64)
    anchors = rng.integers(0, 10**6, size=R).astype(np.int32)
    drafts = rng.integers(0, 10**6, size=(R, K)).astype(np.int32)
    tiers = sorted(set(rng.integers(R, R * (K + 1) + 2, size=6).tolist()))
    cg, kg, ag, dg = to_gpu(conf), to_gpu(cost), to_gpu(anchors), to_gpu(drafts)
    for mode, cap, th, tl in ((dsp.DSP_SCHED_EARLY_STOP, -1, 0.0, None), (dsp.DSP_SCHED_ARGMAX, -1, 0.0, tiers),
                              (dsp.DSP_SCHED_TOP_M, (R * K) // 3, 0.0, None),
                              (dsp.DSP_SCHED_THRESHOLD, -1, 0.3, tiers)):
        print(f"schedule+pack R={R} K={K} mode={mode}", flush=True)
        f = dsp.schedule_pack(cg, kg, ag, dg, mode=mode, max_tokens=cap, threshold=th, tiers=tl)
        s = dsp.schedule_windows(cg, kg, mode=mode, max_tokens=cap, threshold=th)
        p = dsp.pack_ragged(s["windows"], ag, dg, tiers=tl)
        torch.cuda.synchronize()
        for k in ("windows", "survival", "stats"):
            assert torch.equal(f[k], s[k]), k
        T = int(host(p["total_and_tier"])[0])
        for k in ("cu_seqlens", "total_and_tier", "status"):
            assert torch.equal(f[k], p[k]), k
        for k in ("tokens", "row_req", "row_pos"):
            assert torch.equal(f[k][:T], p[k][:T]), k
        o = osch.schedule_windows(conf, cost, mode=mode, max_tokens=cap, threshold=th)
        np.testing.assert_array_equal(host(f["windows"]), o["windows"])
        op = opack.pack_ragged(o["windows"], anchors, drafts, tiers=tl)
        np.testing.assert_array_equal(host(f["tokens"])[:T], op["tokens"])
        assert host(f["total_and_tier"]).tolist() == [op["total"], op["tier"]]
