"""GPU parity of the batched ragged verify (C ABI dsp_verify_rejection) against the oracle."""
import numpy as np
import pytest
import torch

import block_drafting_verification_amd as dsp
import workloads
from oracle import philox as ophilox
from oracle import verify as ov
from parity import (TieCounter, compare_chain_verify, cu_from_windows, dev, host, logits_to_gpu,
                    packed_from_dense, to_gpu, values)

pytestmark = pytest.mark.gpu


def _row_maps(windows, bad=False):
    """The pack's packed-row maps (request, position) for the given windows; with bad=True
    some entries disagree with cu_seqlens (another request, a draft row labelled as an
    anchor, an anchor labelled as a draft row, a request out of range), which the verify
    must detect and resolve by searching cu_seqlens."""
    req = np.concatenate([np.full(w + 1, i, np.int32) for i, w in enumerate(windows)])
    pos = np.concatenate([np.arange(w + 1, dtype=np.int32) for w in windows])
    if bad:
        cu = cu_from_windows(windows)
        drafts = [r for r in range(len(req)) if pos[r] > 0]
        anchors = [int(c) for c in cu[:-1]]
        req[drafts[0]] = (req[drafts[0]] + 1) % len(windows)
        pos[drafts[1]] = 0
        pos[anchors[1]] = 2
        req[drafts[-1]] = -5
    return to_gpu(req), to_gpu(pos)


def _run_case(case, windows, temperature, seed=0, rnd=0, req_id=None, ld_pad=0, want_probs=True,
              row_maps=False):
    R, K, V, dt = case["R"], case["K"], case["V"], case["dtype"]
    tp = packed_from_dense(case["t"], windows)
    if ld_pad:
        tp = np.concatenate([tp, np.zeros((tp.shape[0], ld_pad), dtype=tp.dtype)], axis=1)
    cu = cu_from_windows(windows)
    tg = logits_to_gpu(tp, dt)[:, :V]
    dg = logits_to_gpu(case["d"], dt)
    xg = to_gpu(case["x"].astype(np.int32))
    rid = None if req_id is None else to_gpu(np.asarray(req_id, dtype=np.int64))
    rq, rp = _row_maps(windows, bad=row_maps == "bad") if row_maps else (None, None)
    print(f"verify case R={R} K={K} V={V} dtype={dt} T={temperature} ld={tg.stride(0)} maps={row_maps}",
          flush=True)
    g = dsp.verify_rejection(tg, to_gpu(cu), xg, drf=dg, temperature=temperature, seed=seed, round=rnd,
                             req_id=rid, want_probs=want_probs, row_req=rq, row_pos=rp)
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) == 0
    tv = values(tp[:, :V], dt).astype(np.float64)
    dv = values(case["d"], dt).astype(np.float64)

    def orc(forced):
        return ov.verify_chain(tv, cu, dv, case["x"], temperature, seed=seed, rnd=rnd, req_id=req_id,
                               forced_len=forced)
    return g, orc


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1024, 4099, 40000])
def test_sampled_small(dt, V):
    R, K = 6, 5
    case = workloads.verify_case(R, K, V, dtype=dt, seed=V + (dt == "bf16"), t_sigma=2.0, d_sigma=0.4)
    windows = np.array([5, 0, 3, 5, 1, 4])
    ties = TieCounter()
    for T, maps in ((1.0, False), (0.7, False), (1.0, True)):
        g, orc = _run_case(case, windows, T, seed=11, rnd=2, row_maps=maps)
        compare_chain_verify(g, orc, R, K, windows, ties)
    ties.check()


def test_tiny_verify():
    """4 requests, K=7, V=1024, fp32, Philox seed 0, full windows and a scheduled run."""
    c = workloads.tiny_verify()
    ties = TieCounter()
    g, orc = _run_case(c, np.full(4, 7), 1.0, seed=0)
    compare_chain_verify(g, orc, 4, 7, np.full(4, 7), ties)
    sch = dsp.schedule_windows(to_gpu(c["conf"]), to_gpu(c["cost"]))
    w = host(sch["windows"])
    g, orc = _run_case(c, w, 1.0, seed=0)
    compare_chain_verify(g, orc, 4, 7, w, ties)
    ties.check()


def test_unaligned_rows_and_request_ids():
    R, K, V = 5, 4, 3001
    case = workloads.verify_case(R, K, V, dtype="bf16", seed=5, t_sigma=2.0, d_sigma=0.3)
    windows = np.array([4, 2, 0, 4, 3])
    ties = TieCounter()
    for maps in (False, True, "bad"):
        g, orc = _run_case(case, windows, 1.0, seed=3, rnd=9, req_id=[100, 7, 55, 2**40, 3], ld_pad=3,
                           row_maps=maps)
        compare_chain_verify(g, orc, R, K, windows, ties)
    ties.check()


def test_identical_rows_accept_everything():
    R, K, V = 8, 7, 20000
    case = workloads.verify_case(R, K, V, dtype="bf16", seed=8, t_sigma=3.0, d_sigma=0.0)
    assert np.array_equal(case["d"], case["t"][:, :K])
    g, orc = _run_case(case, np.full(R, K), 1.0, seed=4)
    np.testing.assert_array_equal(host(g["accepted_len"]), K)
    np.testing.assert_array_equal(host(g["out_tokens"])[:, :K], case["x"])
    ties = TieCounter()
    compare_chain_verify(g, orc, R, K, np.full(R, K), ties)
    assert ties.near == 0


def test_greedy_matches_argmax_prefix():
    R, K, V = 12, 6, 30011
    rng = np.random.Generator(np.random.PCG64(3))
    case = workloads.verify_case(R, K, V, dtype="bf16", seed=21, t_sigma=3.0, d_sigma=0.5, temperature=0.0)
    tv = values(case["t"], "bf16")
    am = np.argmax(tv, axis=-1)
    lead = rng.integers(0, K + 1, size=R)
    x = case["x"].copy()
    for i in range(R):
        x[i, :lead[i]] = am[i, :lead[i]]
        if lead[i] < K and x[i, lead[i]] == am[i, lead[i]]:
            x[i, lead[i]] = (x[i, lead[i]] + 1) % V
    case["x"] = x
    windows = np.array([6, 6, 0, 3, 6, 2, 6, 6, 1, 6, 5, 6])
    tp = packed_from_dense(case["t"], windows)
    cu = cu_from_windows(windows)
    g = dsp.verify_rejection(logits_to_gpu(tp, "bf16"), to_gpu(cu), to_gpu(x.astype(np.int32)), temperature=0.0)
    torch.cuda.synchronize()
    o = ov.verify_chain(values(tp, "bf16"), cu, None, x, 0.0)
    np.testing.assert_array_equal(host(g["accepted_len"]), o["accepted_len"])
    np.testing.assert_array_equal(host(g["out_tokens"]), o["out_tokens"])
    np.testing.assert_array_equal(host(g["accepted_len"]), np.minimum(lead, windows))


def test_greedy_ties_lowest_token_and_signed_zero():
    V = 9000
    t = np.full((1, 2, V), -5.0, dtype=np.float32)
    t[0, 0, [4000, 17, 8999]] = 3.0
    t[0, 1, :] = -0.0
    t[0, 1, 5] = 0.0
    tb = workloads.f32_to_bf16_bits(t)
    g = dsp.verify_rejection(to_gpu_bf16_rows(tb[0]), to_gpu(np.array([0, 2], np.int32)),
                             to_gpu(np.array([[17]], np.int32)), temperature=0.0)
    torch.cuda.synchronize()
    assert host(g["accepted_len"])[0] == 1
    assert host(g["out_tokens"])[0].tolist() == [17, 0]


def to_gpu_bf16_rows(bits):
    from parity import to_gpu_bf16
    return to_gpu_bf16(bits)


@pytest.mark.parametrize("dt,V", [("bf16", 5003), ("f32", 5003), ("bf16", 40)])
def test_tree_walk_matches_oracle(dt, V):
    rng = np.random.Generator(np.random.PCG64(31 + V))
    R, N = 6, 20
    tok = np.zeros((R, N), np.int32)
    par = np.zeros((R, N), np.int32)
    rows = []
    nn = rng.integers(1, N + 1, size=R)
    for i in range(R):
        for j in range(N):
            par[i, j] = -1 if j < 3 else rng.integers(-1, j)
        # distinct sibling tokens
        for j in range(N):
            tok[i, j] = rng.integers(0, V)
        r = rng.standard_normal((nn[i] + 1, V)).astype(np.float32) * 3
        # plant a path root -> ... following argmax
        cur = -1
        for _ in range(4):
            kids = [j for j in range(nn[i]) if par[i, j] == cur]
            if not kids:
                break
            j = kids[rng.integers(0, len(kids))]
            sib = [s for s in range(nn[i]) if par[i, s] == cur and s != j]
            while tok[i, j] in tok[i, sib]:
                tok[i, j] = (tok[i, j] + 1) % V
            r[1 + cur, tok[i, j]] = 20.0
            cur = j
        rows.append(workloads.f32_to_bf16_bits(r) if dt == "bf16" else r)
    tp = np.concatenate(rows)
    cu = np.concatenate([[0], np.cumsum(nn + 1)]).astype(np.int32)
    print(f"tree walk R={R} N={N} V={V} dtype={dt}", flush=True)
    g = dsp.verify_rejection(logits_to_gpu(tp, dt), to_gpu(cu), to_gpu(tok), parent=to_gpu(par), temperature=0.0)
    torch.cuda.synchronize()
    o = ov.verify_tree_greedy(values(tp, dt), cu, tok, par)
    np.testing.assert_array_equal(host(g["accepted_len"]), o["accepted_len"])
    np.testing.assert_array_equal(host(g["out_tokens"]), o["out_tokens"])
    np.testing.assert_array_equal(host(g["stop_pos"]), o["stop_node"])
    assert np.all(o["accepted_len"] >= 1)


def test_tree_walk_ties_take_the_lowest_token():
    """Rows of equal values: every arg-max is token 0, so the walk follows the chain of
    children carrying token 0 (the first such child at each node) and the bonus is 0."""
    R, N, V = 2, 6, 999
    par = np.array([[-1, -1, 0, 0, 2, 4], [-1, 0, 1, -1, 3, 4]], np.int32)
    tok = np.array([[5, 0, 0, 3, 0, 0], [0, 0, 7, 4, 1, 2]], np.int32)
    tp = workloads.f32_to_bf16_bits(np.full((R * (N + 1), V), 0.25, np.float32))
    cu = np.array([0, N + 1, 2 * (N + 1)], np.int32)
    g = dsp.verify_rejection(logits_to_gpu(tp, "bf16"), to_gpu(cu), to_gpu(tok), parent=to_gpu(par), temperature=0.0)
    torch.cuda.synchronize()
    o = ov.verify_tree_greedy(values(tp, "bf16"), cu, tok, par)
    np.testing.assert_array_equal(host(g["accepted_len"]), o["accepted_len"])
    np.testing.assert_array_equal(host(g["out_tokens"]), o["out_tokens"])
    np.testing.assert_array_equal(host(g["stop_pos"]), o["stop_node"])
    assert host(g["accepted_len"]).tolist() == [1, 2]


def test_fault_bits_from_bad_tokens_and_windows():
    R, K, V = 3, 4, 2048
    case = workloads.verify_case(R, K, V, dtype="bf16", seed=41)
    x = case["x"].copy()
    x[1, 2] = V + 5
    windows = np.full(R, K)
    tp = packed_from_dense(case["t"], windows)
    g = dsp.verify_rejection(logits_to_gpu(tp, "bf16"), to_gpu(cu_from_windows(windows)), to_gpu(x),
                             drf=logits_to_gpu(case["d"], "bf16"), temperature=1.0)
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) & dsp.DSP_STATUS_TOKEN_RANGE
    acc = host(g["accepted_len"])
    assert acc[1] == -1 and acc[0] >= 0 and acc[2] >= 0
    # a window larger than K
    cu = np.array([0, 5, 10, 16], np.int32)  # last request claims 5 drafts with K = 4
    g = dsp.verify_rejection(logits_to_gpu(tp, "bf16"), to_gpu(cu), to_gpu(case["x"]),
                             drf=logits_to_gpu(case["d"], "bf16"), temperature=1.0)
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) & dsp.DSP_STATUS_WINDOW_RANGE
    assert host(g["accepted_len"])[2] == -1


def test_max_window_64():
    R, K, V = 3, 64, 3000
    case = workloads.verify_case(R, K, V, dtype="bf16", seed=51, t_sigma=1.0, d_sigma=0.05)
    windows = np.array([64, 63, 10])
    ties = TieCounter()
    g, orc = _run_case(case, windows, 1.0, seed=1)
    compare_chain_verify(g, orc, R, K, windows, ties)
    ties.check()


def test_dense_vocab_verify_full():
    """64 requests x K=7 x V=151,936 bf16, full-block windows, T=1: every request checked."""
    c = workloads.dense_verify()
    R, K = c["R"], c["K"]
    ties = TieCounter()
    g, orc = _run_case(c, np.full(R, K), 1.0, seed=0, row_maps=True)
    compare_chain_verify(g, orc, R, K, np.full(R, K), ties)
    ties.check()
    acc = host(g["accepted_len"])
    print("dense verify: mean accepted", acc.mean(), "near ties", ties.near, "of", ties.decisions)


def test_philox_uniforms_bitwise():
    rng = np.random.Generator(np.random.PCG64(77))
    ctr = rng.integers(0, 2**63, size=(5000, 4), dtype=np.uint64)
    ctr[:100] = np.stack([np.full(100, 3), np.arange(100), np.arange(1, 101), np.zeros(100)], axis=1)
    ref = np.stack([ophilox.to_unit_double(w) for w in ophilox.philox4x64_10(ctr, np.array([9, 0], np.uint64)).T], axis=1)
    got = host(dsp.philox_uniforms(to_gpu(ctr.view(np.int64)), 9))
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("T,dt,V", [(1.0, "bf16", 4099), (0.7, "f32", 1024), (0.0, "bf16", 40000)])
def test_cap_accept(T, dt, V):
    """Cap-accept on the full-block packing: the ceiling is the full verify, the committed
    tokens are the compact verify of the cap window (oracle, and the GPU's own compact run)."""
    R, K = 9, 6
    case = workloads.verify_case(R, K, V, dtype=dt, seed=77 + V, t_sigma=2.0, d_sigma=0.4)
    rng = np.random.Generator(np.random.PCG64(V))
    cap = rng.integers(0, K + 2, size=R).astype(np.int32)
    full = np.full(R, K)
    tp = packed_from_dense(case["t"], full)
    cu = cu_from_windows(full)
    tg, dg, xg = logits_to_gpu(tp, dt)[:, :V], logits_to_gpu(case["d"], dt), to_gpu(case["x"].astype(np.int32))
    print(f"cap-accept R={R} K={K} V={V} dtype={dt} T={T}", flush=True)
    g = dsp.verify_rejection(tg, to_gpu(cu), xg, drf=dg, temperature=T, seed=4, round=2, cap=to_gpu(cap))
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) == 0
    tv = values(tp[:, :V], dt).astype(np.float64)
    dv = values(case["d"], dt).astype(np.float64)
    ceil_g = host(g["ceiling"]).astype(np.int64)
    own = ov.verify_chain(tv, cu, dv, case["x"], T, seed=4, rnd=2, cap=cap)
    ties = TieCounter()
    for i in np.nonzero(ceil_g != own["ceiling"])[0]:
        k = int(min(ceil_g[i], own["ceiling"][i])) + 1
        assert own["accept_margin"][i, k - 1] < 1e-6, (i, ceil_g[i], own["ceiling"][i])
        ties.near += 1
    rep = own if ties.near == 0 else ov.verify_chain(tv, cu, dv, case["x"], T, seed=4, rnd=2, cap=cap,
                                                     forced_len=ceil_g)
    ties.decisions += int(own["ceiling"].sum()) + R
    acc, toks = host(g["accepted_len"]).astype(np.int64), host(g["out_tokens"]).astype(np.int64)
    np.testing.assert_array_equal(acc, rep["accepted_len"])
    np.testing.assert_array_equal(acc, np.minimum(ceil_g, np.minimum(cap, K)))
    for i in range(R):
        np.testing.assert_array_equal(toks[i, :acc[i]], rep["out_tokens"][i, :acc[i]])
        if toks[i, acc[i]] != rep["out_tokens"][i, acc[i]]:
            assert rep["sample_margin"][i] < 1e-6
            ties.near += 1
        assert np.all(toks[i, acc[i] + 1:] == -1)
    ties.check()
    # the GPU's own compact verify of the cap window commits the same tokens
    c = np.minimum(cap, K)
    tpc = packed_from_dense(case["t"], c)
    gc = dsp.verify_rejection(logits_to_gpu(tpc, dt)[:, :V], to_gpu(cu_from_windows(c)), xg, drf=dg, temperature=T,
                              seed=4, round=2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(gc["accepted_len"]), host(g["accepted_len"]))
    np.testing.assert_array_equal(host(gc["out_tokens"]), host(g["out_tokens"]))


def test_scheduled_ragged_verify_full():
    """The confidence-scheduled ragged verify workload: 256 requests x K=16, V=151,936 bf16;
    scheduler -> pack -> compact verify on the GPU, every request checked against the oracle."""
    c = workloads.scheduled_verify()
    R, K, V = c["R"], c["K"], c["V"]
    sch = dsp.schedule_windows(to_gpu(c["conf"]), to_gpu(c["cost"]))
    xg = to_gpu(c["x"].astype(np.int32))
    pk = dsp.pack_ragged(sch["windows"], to_gpu(c["anchors"]), xg)
    w = host(sch["windows"])
    tp = packed_from_dense(c["t"], w)
    print(f"scheduled verify R={R} K={K} V={V} packed rows={tp.shape[0]} drafts={int(w.sum())}", flush=True)
    g = dsp.verify_rejection(logits_to_gpu(tp, "bf16"), pk["cu_seqlens"], xg, drf=logits_to_gpu(c["d"], "bf16"),
                             temperature=1.0, seed=0, round=3, row_req=pk["row_req"], row_pos=pk["row_pos"])
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) == 0
    cu = cu_from_windows(w)
    np.testing.assert_array_equal(host(pk["cu_seqlens"]), cu)
    tv = values(tp, "bf16").astype(np.float64)
    dv = values(c["d"], "bf16").astype(np.float64)

    def orc(forced):
        return ov.verify_chain(tv, cu, dv, c["x"], 1.0, seed=0, rnd=3, forced_len=forced)
    ties = TieCounter()
    compare_chain_verify(g, orc, R, K, w, ties)
    ties.check()


def test_scheduled_verify_captured_at_full_size():
    """The same scheduled batch verified with max_rows = R x (K+1) = 4,352 rows while only the
    packed rows at the front are live (one graph captured for the largest batch): past 16,384
    items the statistics pass runs a capped grid of workgroups that loop over the items and
    stop at the device-side packed total. Outputs must equal the exact-size call bit for bit,
    with the pack's row maps and with the binary search of cu_seqlens."""
    c = workloads.scheduled_verify()
    R, K, V = c["R"], c["K"], c["V"]
    sch = dsp.schedule_windows(to_gpu(c["conf"]), to_gpu(c["cost"]))
    xg = to_gpu(c["x"].astype(np.int32))
    pk = dsp.pack_ragged(sch["windows"], to_gpu(c["anchors"]), xg)
    w = host(sch["windows"])
    tp = packed_from_dense(c["t"], w)
    T = tp.shape[0]
    full = R * (K + 1)
    tg_exact = logits_to_gpu(tp, "bf16")
    tg_full = torch.zeros(full, V, dtype=torch.bfloat16, device=tg_exact.device)
    tg_full[:T].copy_(tg_exact)
    dg = logits_to_gpu(c["d"], "bf16")
    print(f"full-size capture: packed rows {T} of {full}, items {full * 20}", flush=True)
    keys = ("accepted_len", "out_tokens", "stop_pos", "p_x", "q_x")
    for maps in (True, False):
        extra = dict(row_req=pk["row_req"], row_pos=pk["row_pos"]) if maps else {}
        ref = dsp.verify_rejection(tg_exact, pk["cu_seqlens"], xg, drf=dg, temperature=1.0, seed=0, round=5, **extra)
        got = dsp.verify_rejection(tg_full, pk["cu_seqlens"], xg, drf=dg, temperature=1.0, seed=0, round=5,
                                   max_rows=full, **extra)
        torch.cuda.synchronize()
        assert int(host(got["status"])[0]) == 0 and int(host(ref["status"])[0]) == 0
        for k in keys:
            assert torch.equal(got[k], ref[k]), (maps, k)


def test_masked_vocabulary_entries():
    """Rows with -inf entries (a masked or padded vocabulary, same mask for target and draft):
    the masked tokens carry no probability mass on either side and are never drawn."""
    R, K, V = 6, 5, 5003
    case = workloads.verify_case(R, K, V, dtype="bf16", seed=91, t_sigma=2.0, d_sigma=0.4)
    rng = np.random.default_rng(4)
    mask = rng.random(V) < 0.15
    mask[-3:] = True  # a padded tail
    t, d = case["t"].copy(), case["d"].copy()
    t[..., mask] = 0xFF80  # bf16 -inf
    d[..., mask] = 0xFF80
    d32 = workloads.bf16_bits_to_f32(d)
    x = np.argmax(d32, axis=-1).astype(np.int32)  # a most likely (unmasked) draft token
    case = dict(case, t=t, d=d, x=x)
    windows = np.array([5, 0, 3, 5, 1, 4])
    ties = TieCounter()
    for T in (1.0, 0.7):
        g, orc = _run_case(case, windows, T, seed=13, rnd=1, row_maps=True)
        compare_chain_verify(g, orc, R, K, windows, ties)
        toks = host(g["out_tokens"])
        assert not np.any(mask[toks[toks >= 0]]), "a masked token was drawn"
    ties.check()


def test_scheduled_workload_static_full_windows():
    """The static run of the scheduled ragged verify workload: 256 requests x 16 full windows,
    8,448 packed target rows of V=151,936 bf16 (2.567 GB with the draft rows); every request
    checked against the oracle (float32 values are passed: bf16 widens exactly)."""
    c = workloads.scheduled_verify()
    R, K, V = c["R"], c["K"], c["V"]
    w = np.full(R, K)
    tp = c["t"].reshape(R * (K + 1), V)
    cu = cu_from_windows(w)
    xg = to_gpu(c["x"].astype(np.int32))
    print(f"static verify R={R} K={K} V={V} packed rows={tp.shape[0]}", flush=True)
    rq = to_gpu(np.repeat(np.arange(R, dtype=np.int32), K + 1))
    rp = to_gpu(np.tile(np.arange(K + 1, dtype=np.int32), R))
    g = dsp.verify_rejection(logits_to_gpu(tp, "bf16"), to_gpu(cu), xg, drf=logits_to_gpu(c["d"], "bf16"),
                             temperature=1.0, seed=0, round=4, row_req=rq, row_pos=rp)
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) == 0
    tv = values(tp, "bf16")
    dv = values(c["d"], "bf16")

    def orc(forced):
        return ov.verify_chain(tv, cu, dv, c["x"], 1.0, seed=0, rnd=4, forced_len=forced)
    ties = TieCounter()
    compare_chain_verify(g, orc, R, K, w, ties)
    ties.check()
    acc = host(g["accepted_len"])
    print("static verify: mean accepted", acc.mean(), "near ties", ties.near, "of", ties.decisions)
