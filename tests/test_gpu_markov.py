"""GPU parity of the Markov-head chain and PCTree expansion against the oracle."""
import numpy as np
import pytest
import torch

import block_drafting_verification_amd as dsp
import workloads
from oracle import markov as om
from oracle import pctree as opt
from oracle import verify as ov
from parity import ARGMAX_BAND, SAMPLE_BAND, TieCounter, host, to_gpu, to_gpu_bf16, to_gpu_bf16_token_major

pytestmark = pytest.mark.gpu


def _gpu_inputs(c, token_major=False):
    Wt = np.ascontiguousarray(c["W"].T)  # second factor stored vocab-major
    Lg = to_gpu_bf16_token_major(c["L"]) if token_major else to_gpu_bf16(c["L"])
    return (Lg, to_gpu_bf16(c["U"]), to_gpu_bf16(Wt), to_gpu(c["anchors"].astype(np.int32)))


def _f32(c):
    return (workloads.bf16_bits_to_f32(c["L"]), workloads.bf16_bits_to_f32(c["U"]),
            workloads.bf16_bits_to_f32(c["W"]))


def _check_chain(c, requests=None, want_logq=True, w_boost=1.0, token_major=False):
    L, U, W = _f32(c)
    if w_boost != 1.0:
        Wb = workloads.f32_to_bf16_bits(W * np.float32(w_boost))
        c = dict(c, W=Wb)
        L, U, W = _f32(c)
    Lg, Ug, Wtg, ag = _gpu_inputs(c, token_major)
    print(f"chain R={c['R']} B={c['B']} V={c['V']} rank={c['rank']} token_major={token_major}", flush=True)
    g = dsp.draft_markov_step(Lg, Ug, Wtg, ag, want_logq=want_logq)
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) == 0
    y = host(g["y"]).astype(np.int64)
    sel = np.arange(c["R"]) if requests is None else np.asarray(requests)
    orc = om.chain(L[sel], U, W, c["anchors"][sel], forced=y[sel])
    ties = TieCounter()
    ties.decisions += y[sel].size
    mism = np.argwhere(orc["y"] != y[sel])
    for ii, d in mism:
        i = sel[ii]
        prev = c["anchors"][i] if d == 0 else y[i, d - 1]
        z = om.markov_logits(L[i, d][None], U, W, [prev])[0]
        gap = z[orc["y"][ii, d]] - z[y[i, d]]
        assert gap < ARGMAX_BAND * max(1.0, abs(z[orc["y"][ii, d]])), (i, d, gap)
        ties.near += 1
    ties.check()
    if want_logq:
        lq = host(g["logq"]).astype(np.float64)[sel]
        np.testing.assert_allclose(lq, orc["logq_forced"], rtol=1e-5, atol=1e-5)
    return y


@pytest.mark.parametrize("R,B,V,rank", [(5, 4, 1000, 32), (130, 3, 4099, 64), (7, 5, 30000, 256),
                                        (300, 2, 129, 96), (3, 2, 2000, 512), (600, 2, 9000, 128)])
def test_chain_small(R, B, V, rank):
    c = workloads.markov_case(R, B, V, rank=rank, seed=R + V)
    _check_chain(c, w_boost=300.0)  # a Markov term large enough to change choices
    _check_chain(c)
    _check_chain(c, want_logq=False, w_boost=300.0)  # arg-max only
    dsp.set_option("chain_sched", 1)  # the opt-in scheduled GEMM (rank up to 256)
    try:
        _check_chain(c, want_logq=False, w_boost=300.0)
    finally:
        dsp.set_option("chain_sched", 0)


def test_chain_of_course_fixture():
    import json, os
    gpath = os.path.join(os.path.dirname(__file__), "golden", "of_course_markov.json")
    g = json.load(open(gpath))
    V, r = g["vocab"], 32
    L = np.array(g["L"], np.float32)[None]
    U = np.zeros((V, r), np.float32)
    U[:, :2] = np.array(g["U"], np.float32)
    W = np.zeros((r, V), np.float32)
    W[:2] = np.array(g["W"], np.float32)
    c = dict(L=workloads.f32_to_bf16_bits(L), U=workloads.f32_to_bf16_bits(U), W=workloads.f32_to_bf16_bits(W),
             anchors=np.array([g["tokens"]["anchor"]], np.int32), R=1, B=2, V=V, rank=r)
    y = _check_chain(c)
    inv = {v: k for k, v in g["tokens"].items()}
    assert [inv[int(t)] for t in y[0]] == g["expected_with_markov"]


def test_chain_c4_full():
    """256 requests x 16 steps, V=151,936, rank 256; every request checked with replay."""
    c = workloads.markov_chain()
    _check_chain(c, want_logq=True)


@pytest.mark.parametrize("R,B,V", [(8, 4, 1000), (136, 3, 4099), (264, 2, 30011)])
def test_chain_token_major_layout(R, B, V):
    """Base logits stored token-major ([B, V, R]): tokens exact against the oracle (counted
    near-ties), and every output bit-identical to the row-major call's (same arithmetic)."""
    c = workloads.markov_case(R, B, V, rank=256, seed=R + V + 7)
    y = _check_chain(c, w_boost=300.0, token_major=True)
    Lr, Ug, Wtg, ag = _gpu_inputs(c)
    Lt = _gpu_inputs(c, True)[0]
    assert Lt.stride(0) == 1
    a = dsp.draft_markov_step(Lr, Ug, Wtg, ag, want_logq=True)  # both on the per-step kernels
    b = dsp.draft_markov_step(Lt, Ug, Wtg, ag, want_logq=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(a["y"]), host(b["y"]))
    np.testing.assert_array_equal(host(a["logq"]).view(np.uint32), host(b["logq"]).view(np.uint32))
    assert int(host(b["status"])[0]) == 0


def test_chain_token_major_c4_full():
    """The Markov-chain workload (256 x 16, V=151,936, rank 256) with token-major base
    logits: every request against the oracle, and identical to the row-major outputs."""
    c = workloads.markov_chain()
    y = _check_chain(c, want_logq=True, token_major=True)
    Lr, Ug, Wtg, ag = _gpu_inputs(c)
    a = dsp.draft_markov_step(Lr, Ug, Wtg, ag)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(a["y"]), y)


def _padded_l(bits, vp):
    """[R, B, V] base logits in a buffer whose rows are vp >= V entries apart (vp a
    multiple of 8: the persistent chain's alignment)."""
    R, B, V = bits.shape
    buf = np.zeros((R, B, vp), np.uint16)
    buf[..., :V] = bits
    return to_gpu_bf16(buf)[..., :V]


def _chain_both_paths(c, Lg, want_logq=True):
    """The chain on both launch paths; checks that the persistent one ran, that the tokens
    are identical and that log q agrees to fp32 rounding (the paths split the vocabulary
    into different partial sums)."""
    _, Ug, Wtg, ag = _gpu_inputs(c)
    dsp.prof_reset()
    dsp.prof_enable(kernels=["CHAIN_PERSIST"])
    dsp.set_option("chain_persistent", 1)
    try:
        p = dsp.draft_markov_step(Lg, Ug, Wtg, ag, want_logq=want_logq)
        torch.cuda.synchronize()
        assert dsp.prof_query("CHAIN_PERSIST")[1] == 1, "the persistent chain did not run"
    finally:
        dsp.set_option("chain_persistent", 0)
        dsp.prof_enable(False)
        dsp.prof_reset()
    q = dsp.draft_markov_step(Lg, Ug, Wtg, ag, want_logq=want_logq)
    torch.cuda.synchronize()
    assert int(host(p["status"])[0]) == 0 and int(host(q["status"])[0]) == 0
    np.testing.assert_array_equal(host(p["y"]), host(q["y"]))
    return p, q


@pytest.mark.parametrize("R,B,V", [(1, 3, 100), (5, 4, 1000), (33, 2, 4099), (100, 3, 30011), (256, 2, 9000),
                                   (64, 3, 151936), (256, 2, 155000)])
def test_chain_persistent(R, B, V):
    """Rank 256, aligned row-major L: the whole chain in one persistent launch, against the
    oracle (every request, counted near-ties) and against the per-step launches.
    Covers one row, ragged column blocks, few vocabulary tiles (idle waves and workgroups)
    and the largest vocabulary the path takes (19 tiles per workgroup)."""
    c = workloads.markov_case(R, B, V, rank=256, seed=R + V + 11)
    c = dict(c, W=workloads.f32_to_bf16_bits(_f32(c)[2] * np.float32(300.0)))  # choices the head changes
    vp = (V + 7) // 8 * 8
    Lg = _padded_l(c["L"], vp)
    print(f"persistent chain R={R} B={B} V={V}", flush=True)
    p, q = _chain_both_paths(c, Lg)
    L, U, W = _f32(c)
    y = host(p["y"]).astype(np.int64)
    orc = om.chain(L, U, W, c["anchors"], forced=y)
    ties = TieCounter()
    ties.decisions += y.size
    for i, d in np.argwhere(orc["y"] != y):
        prev = c["anchors"][i] if d == 0 else y[i, d - 1]
        z = om.markov_logits(L[i, d][None], U, W, [prev])[0]
        assert z[orc["y"][i, d]] - z[y[i, d]] < ARGMAX_BAND * max(1.0, abs(z[orc["y"][i, d]])), (i, d)
        ties.near += 1
    ties.check()
    for name, g in (("persistent", p), ("per step", q)):
        lq = host(g["logq"]).astype(np.float64)
        err = np.abs(lq - orc["logq_forced"])
        bad = np.argwhere(err > 1e-5 + 1e-5 * np.abs(orc["logq_forced"]))
        assert not len(bad), (name, [(int(i), int(d), lq[i, d], orc["logq_forced"][i, d]) for i, d in bad[:5]])


def test_chain_persistent_c4_matches_per_step():
    """The Markov-chain workload (256 x 16, V=151,936): persistent and per-step launches
    give identical tokens and matching log q (oracle parity of this shape: test_chain_c4_full)."""
    c = workloads.markov_chain()
    Lg, _, _, _ = _gpu_inputs(c)
    _chain_both_paths(c, Lg, want_logq=True)
    _chain_both_paths(c, Lg, want_logq=False)


def test_chain_persistent_barrier_timeout_is_reported():
    """A grid barrier that gives up (forced from the host with a spin limit of 0 polls)
    sets DSP_STATUS_TIMEOUT and the launch still drains; the next call, with the default
    limit, is correct."""
    c = workloads.markov_case(64, 3, 9000, rank=256, seed=77)
    Lg, Ug, Wtg, ag = _gpu_inputs(c)
    dsp.set_option("spin_limit", 0)
    dsp.set_option("chain_persistent", 1)
    try:
        g = dsp.draft_markov_step(Lg, Ug, Wtg, ag)
        torch.cuda.synchronize()
    finally:
        dsp.set_option("spin_limit", 1 << 20)
        dsp.set_option("chain_persistent", 0)
    assert int(host(g["status"])[0]) & dsp.DSP_STATUS_TIMEOUT
    _chain_both_paths(c, Lg)


def _check_tree(c, topk, F, N, requests=None, w_boost=1.0, status=0):
    """Tree against the oracle, node by node for every checked request: the oracle replays the
    GPU's tree at near-tie cuts only (counted) and otherwise expands on its own; tokens,
    parents, depths and ancestor masks must then be equal, scores within 1e-5."""
    L, U, W = _f32(c)
    if w_boost != 1.0:
        c = dict(c, W=workloads.f32_to_bf16_bits(W * np.float32(w_boost)))
        L, U, W = _f32(c)
    Lg, Ug, Wtg, ag = _gpu_inputs(c)
    print(f"tree R={c['R']} D={c['B']} V={c['V']} k={topk} F={F} N={N}", flush=True)
    g = dsp.tree_expand(Lg, Ug, Wtg, ag, topk, F, N, want_mask=True)
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) == status
    gm = host(g["anc_mask"]).view(np.uint64)
    sel = list(range(c["R"])) if requests is None else list(requests)
    gt, gp, gd, gs, gn = (host(g[k]) for k in ("node_token", "node_parent", "node_depth", "node_score", "n_nodes"))
    o = opt.tree_expand(L, U.astype(np.float64), W.astype(np.float64), c["anchors"], topk, F, N, requests=sel,
                        prefer=(gt, gp, gn), band=ARGMAX_BAND)
    om_mask = opt.ancestor_masks(o["node_parent"], o["n_nodes"])
    ties = TieCounter()
    for i in sel:
        ties.decisions += int(o["decisions"][i])
        ties.near += int(o["replays"][i])
        if o["replays"][i]:
            ties.notes.append(("tree", i, int(o["replays"][i])))
        assert gn[i] == o["n_nodes"][i], i
        n = gn[i]
        np.testing.assert_array_equal(gt[i], o["node_token"][i], err_msg=f"request {i} tokens")
        np.testing.assert_array_equal(gp[i], o["node_parent"][i], err_msg=f"request {i} parents")
        np.testing.assert_array_equal(gd[i], o["node_depth"][i], err_msg=f"request {i} depths")
        np.testing.assert_allclose(gs[i, :n], o["node_score"][i, :n], rtol=1e-5, atol=1e-5)
        np.testing.assert_array_equal(gm[i], om_mask[i])  # tree-causal ancestor masks, exact
    print(f"  near-ties replayed: {ties.near} of {ties.decisions} cut decisions", flush=True)
    ties.check()
    return g


@pytest.mark.parametrize("R,D,V,k,F,N,rank", [(3, 4, 700, 2, 3, 8, 32), (9, 6, 5003, 4, 16, 64, 64),
                                              (2, 3, 40000, 4, 16, 20, 256), (140, 2, 300, 3, 5, 7, 32),
                                              (20, 3, 40000, 4, 16, 30, 64), (3, 8, 3000, 4, 16, 100, 32)])
def test_tree_small(R, D, V, k, F, N, rank):
    c = workloads.markov_case(R, D, V, rank=rank, seed=7 * R + V)
    _check_tree(c, k, F, N, w_boost=200.0)
    _check_tree(c, k, F, N)


def test_tree_k1_f1_is_chain():
    c = workloads.markov_case(4, 5, 3000, rank=64, seed=99)
    Lg, Ug, Wtg, ag = _gpu_inputs(c)
    t = dsp.tree_expand(Lg, Ug, Wtg, ag, 1, 1, 5)
    ch = dsp.draft_markov_step(Lg, Ug, Wtg, ag)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(t["node_token"]), host(ch["y"]))
    np.testing.assert_array_equal(host(t["node_parent"]), np.tile(np.arange(-1, 4), (4, 1)))


def test_tree_c5_sampled_requests():
    """128 requests, depth 16, V=129,280, k=4, F=16, N=64: 32 requests spread over the batch
    checked node by node against the oracle."""
    c = workloads.markov_case(128, 16, workloads.V_DSV4, 256, seed=1005)
    g = _check_tree(c, 4, 16, 64, requests=list(range(0, 128, 4)))
    n = host(g["n_nodes"])
    assert np.all(n == 64)


def test_tree_verify_c5_shape_planted_paths():
    """Tree verify on targets shaped like the PCTree workload with a planted accepted path per request."""
    c = workloads.markov_case(8, 16, workloads.V_DSV4, 256, seed=1005)
    Lg, Ug, Wtg, ag = _gpu_inputs(c)
    t = dsp.tree_expand(Lg, Ug, Wtg, ag, 4, 16, 64)
    torch.cuda.synchronize()
    tok, par = host(t["node_token"]), host(t["node_parent"])
    R, N, V = 8, 64, workloads.V_DSV4
    tgt = workloads.tree_target(R, N + 1, V, seed=77)
    tgt32 = workloads.bf16_bits_to_f32(tgt).copy()
    rng = np.random.Generator(np.random.PCG64(5))
    planted = []
    for i in range(R):
        depth = int(rng.integers(0, 8))
        cur, n = -1, 0
        while n < depth:
            kids = np.flatnonzero(par[i] == cur)
            if kids.size == 0:
                break
            j = int(kids[0])
            tgt32[i, 1 + cur, tok[i, j]] = 50.0
            cur = j
            n += 1
        planted.append(n)
    tb = workloads.f32_to_bf16_bits(tgt32).reshape(R * (N + 1), V)
    cu = (np.arange(R + 1) * (N + 1)).astype(np.int32)
    g = dsp.verify_rejection(to_gpu_bf16(tb), to_gpu(cu), t["node_token"], parent=t["node_parent"], temperature=0.0)
    torch.cuda.synchronize()
    o = ov.verify_tree_greedy(workloads.bf16_bits_to_f32(tb), cu, tok, par)
    np.testing.assert_array_equal(host(g["accepted_len"]), o["accepted_len"])
    np.testing.assert_array_equal(host(g["out_tokens"]), o["out_tokens"])
    assert np.all(o["accepted_len"] >= np.array(planted))


# ---------------------------------------------------------------- sampled chain

def _check_sampled(c, T, seed=0, rnd=0, requests=None, w_boost=1.0, token_major=False):
    """Sampled chain against the oracle with replay of the GPU's draws: the emitted bf16 rows
    bit-exact except entries the oracle marks as rounding near-ties (then within one bf16
    unit), the draws exact except counted near-ties, logq within 1e-5."""
    L, U, W = _f32(c)
    if w_boost != 1.0:
        c = dict(c, W=workloads.f32_to_bf16_bits(W * np.float32(w_boost)))
        L, U, W = _f32(c)
    Lg, Ug, Wtg, ag = _gpu_inputs(c, token_major)
    print(f"sampled chain R={c['R']} B={c['B']} V={c['V']} rank={c['rank']} T={T} token_major={token_major}",
          flush=True)
    g = dsp.draft_markov_sample(Lg, Ug, Wtg, ag, T, seed=seed, round=rnd)
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) == 0
    y = host(g["y"]).astype(np.int64)
    sel = np.arange(c["R"]) if requests is None else np.asarray(requests)
    zg = workloads.bf16_bits_to_f32(host(g["z"][sel].contiguous().view(torch.int16)).view(np.uint16))
    orc = om.chain_sampled(L[sel], U, W, c["anchors"][sel], T, seed=seed, rnd=rnd, req_id=sel, forced=y[sel])
    # emitted rows
    diff = zg.astype(np.float64) != orc["zhat"]
    assert not np.any(diff & ~orc["round_tie"]), np.argwhere(diff & ~orc["round_tie"])[:5]
    if diff.any():
        # an fp32 value near a rounding midpoint lands within one unit plus the fp32 band
        # (near zero, after cancellation, the band spans several units)
        zo = orc["zhat"][diff]
        _, _, ulp = om.round_bf16(zo)
        allow = ulp * 1.0000001 + om.ROUND_BAND * np.maximum(1.0, np.abs(zo))
        assert np.all(np.abs(zg[diff] - zo) <= allow)
    # draws
    ties = TieCounter()
    ties.decisions += y[sel].size
    for ii, d in np.argwhere(orc["y"] != y[sel]):
        band = SAMPLE_BAND + orc["tie_shift"][ii, d]
        assert orc["sample_margin"][ii, d] < band, (sel[ii], d, orc["sample_margin"][ii, d], band)
        ties.near += 1
        ties.notes.append((int(sel[ii]), int(d)))
    ties.check()
    # logq: 1e-5, widened where rounding near-ties may have moved the drawn token's own
    # rounded value (tok_dev / T) or the row's normaliser (by a factor within 1 / (1 - eps))
    lq = host(g["logq"]).astype(np.float64)[sel]
    allow = (1e-5 * np.maximum(1.0, np.abs(orc["logq_forced"])) + orc["tok_dev"] / T
             - np.log1p(-np.minimum(orc["eps"], 0.5)))
    err = np.abs(lq - orc["logq_forced"])
    assert np.all(err <= allow), (np.argwhere(err > allow)[:5], err.max())
    return g, y


@pytest.mark.parametrize("R,B,V,rank,T", [(5, 4, 1000, 32, 1.0), (130, 3, 4099, 64, 0.7), (7, 3, 30000, 256, 1.3),
                                          (300, 2, 129, 96, 1.0), (3, 2, 2000, 512, 0.5)])
def test_chain_sampled_small(R, B, V, rank, T):
    c = workloads.markov_case(R, B, V, rank=rank, seed=R + V + 1)
    _check_sampled(c, T, seed=3, rnd=1, w_boost=100.0)
    _check_sampled(c, T, seed=4, rnd=2)


def test_chain_sampled_token_major_layout():
    """Sampled chain from token-major base logits: oracle parity, and the draws, logq and
    emitted rows bit-identical to the row-major call's."""
    c = workloads.markov_case(40, 3, 9001, rank=256, seed=41)
    g, y = _check_sampled(c, 0.8, seed=5, rnd=3, w_boost=100.0, token_major=True)
    Lr, Ug, Wtg, ag = _gpu_inputs(dict(c, W=workloads.f32_to_bf16_bits(_f32(c)[2] * np.float32(100.0))))
    a = dsp.draft_markov_sample(Lr, Ug, Wtg, ag, 0.8, seed=5, round=3)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(a["y"]), y)
    np.testing.assert_array_equal(host(a["logq"]).view(np.uint32), host(g["logq"]).view(np.uint32))
    np.testing.assert_array_equal(host(a["z"].contiguous().view(torch.int16)), host(g["z"].contiguous().view(torch.int16)))


def test_chain_sampled_round_dev_and_req_id():
    """A device round equals the same host round; request ids move the uniforms."""
    c = workloads.markov_case(6, 3, 2000, rank=32, seed=12)
    Lg, Ug, Wtg, ag = _gpu_inputs(c)
    a = dsp.draft_markov_sample(Lg, Ug, Wtg, ag, 1.0, seed=9, round=5)
    rd = torch.full((1,), 5, dtype=torch.int64, device=Lg.device)
    b = dsp.draft_markov_sample(Lg, Ug, Wtg, ag, 1.0, seed=9, round=0, round_dev=rd)
    rid = torch.arange(100, 106, dtype=torch.int64, device=Lg.device)
    e = dsp.draft_markov_sample(Lg, Ug, Wtg, ag, 1.0, seed=9, round=5, req_id=rid)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(a["y"]), host(b["y"]))
    assert int(host(rd)[0]) == 5  # read, not advanced
    L, U, W = _f32(c)
    o = om.chain_sampled(L, U, W, c["anchors"], 1.0, seed=9, rnd=5, req_id=np.arange(100, 106),
                         forced=host(e["y"]).astype(np.int64))
    bad = np.argwhere(o["y"] != host(e["y"]))
    assert all(o["sample_margin"][i, d] < SAMPLE_BAND + o["tie_shift"][i, d] for i, d in bad)


def test_chain_sampled_c4_shape():
    """The Markov-chain workload's shape (256 x 16, V=151,936, rank 256), sampled at T=1;
    6 requests checked against the oracle through all 16 steps."""
    c = workloads.markov_chain()
    _check_sampled(c, 1.0, seed=0, rnd=0, requests=[0, 1, 77, 128, 200, 255])


def test_chain_and_tree_masked_vocabulary():
    """-inf base logits (a masked vocabulary): never chosen by the chain, the sampled chain or
    the tree, and no mass in the log-sum-exp."""
    c = workloads.markov_case(5, 3, 3001, rank=64, seed=33)
    rng = np.random.default_rng(5)
    mask = rng.random(3001) < 0.2
    L = c["L"].copy()
    L[..., mask] = 0xFF80
    c = dict(c, L=L)
    y = _check_chain(c, want_logq=True)
    assert not np.any(mask[y])
    g, ys = _check_sampled(c, 1.0, seed=2, rnd=0)
    assert not np.any(mask[ys])
    t = _check_tree(c, 4, 8, 16)
    nt = host(t["node_token"])
    assert not np.any(mask[nt[nt >= 0]])


@pytest.mark.parametrize("R,F,depth", [(5, 16, 0), (40, 16, 0), (40, 16, 2), (5, 16, 2)])
def test_tree_too_few_finite_entries_is_a_fault(R, F, depth):
    """Request 0's base logits at one depth are masked but for two tokens, fewer than k = 4:
    a fault (status bit) on both of the GEMM's paths -- blocks of at most 16 requests add the
    base logits through the matrix cores (R = 5 at depth 1; 16 parents per request at depth
    3), the others per row. Every other request still matches the oracle."""
    c = workloads.markov_case(R, 3, 3001, rank=64, seed=100 + R + depth)
    L = c["L"].copy()
    keep = np.zeros(3001, dtype=bool)
    keep[[17, 2900]] = True
    L[0, depth, ~keep] = 0xFF80
    c = dict(c, L=L)
    _check_tree(c, 4, F, 24, requests=range(1, R), status=dsp.DSP_STATUS_NONFINITE)


def _tree_exact(c, topk, F, N):
    """Tree against the oracle with no near-tie allowance (cases whose ties the order rules
    settle exactly)."""
    L, U, W = _f32(c)
    Lg, Ug, Wtg, ag = _gpu_inputs(c)
    print(f"tree (exact) R={c['R']} D={c['B']} V={c['V']} k={topk} F={F} N={N}", flush=True)
    g = dsp.tree_expand(Lg, Ug, Wtg, ag, topk, F, N)
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) == 0
    o = opt.tree_expand(L, U, W, c["anchors"], topk, F, N)
    for k in ("node_token", "node_parent", "node_depth", "n_nodes"):
        np.testing.assert_array_equal(host(g[k]), o[k], err_msg=k)
    np.testing.assert_allclose(host(g["node_score"]), o["node_score"], rtol=1e-5, atol=1e-5)
    return g, o


@pytest.mark.parametrize("lval", [0.0, 1.5])
def test_tree_all_equal_rows(lval):
    """Every z equal (constant base logits, zero Markov factors): children are the lowest ids,
    the frontier follows (parent slot, child rank). Every candidate sits exactly on the row
    bound's probe values, the tightest case for the selection's lower bound."""
    c = workloads.markov_case(3, 4, 2000, rank=32, seed=41)
    c["L"][:] = workloads.f32_to_bf16_bits(np.full(c["L"].shape, lval, dtype=np.float32))
    c["U"][:] = 0
    c["W"][:] = 0
    g, o = _tree_exact(c, 4, 8, 20)
    assert set(host(g["node_token"])[0, :4]) == {0, 1, 2, 3}


def test_tree_planted_top4_at_probe_tokens():
    """Each base-logit row has its four largest values at the probe tokens (one per 256-token
    block class, 1 block apart), so the children's 4th-largest z equals the row bound's
    smallest probe value up to the margin."""
    c = workloads.markov_case(4, 5, 3001, rank=64, seed=42, l_sigma=1.0)
    Lf = workloads.bf16_bits_to_f32(c["L"])
    for t, val in ((7, 20.0), (300, 19.0), (600, 18.5), (900, 18.0)):
        Lf[:, :, t] = val
    c["L"] = workloads.f32_to_bf16_bits(Lf)
    g, o = _tree_exact(c, 4, 4, 16)
    tok, dep = host(g["node_token"]), host(g["node_depth"])
    for i in range(c["R"]):
        assert set(tok[i][dep[i] == 1]) == {7, 300, 600, 900}


def test_tree_tiny_vocabulary():
    """V = 5 (one 256-token block: three probe classes empty, no row bound)."""
    c = workloads.markov_case(3, 3, 5, rank=32, seed=43)
    _check_tree(c, 4, 4, 12)


def test_tree_depth_one():
    """D = 1: one expansion of the anchors (no probe pass, no row bound)."""
    c = workloads.markov_case(5, 1, 4001, rank=64, seed=44)
    _check_tree(c, 4, 4, 4)
    _check_tree(c, 3, 2, 2, w_boost=200.0)


def test_tree_verify_on_pctree_workload_target():
    """Greedy tree verify on the PCTree workload's own target (128 requests x 65 rows of
    V=129,280 bf16 laid out root first) over the GPU's own 128 x 64-node trees: every request
    checked against the oracle's walk; a second pass plants an accepted path of random depth in
    each request's rows."""
    c = workloads.pctree()
    R, N, V = c["R"], c["topN"], c["V"]
    Lg, Ug, Wtg, ag = _gpu_inputs(c)
    t = dsp.tree_expand(Lg, Ug, Wtg, ag, c["topk"], c["frontier"], N)
    torch.cuda.synchronize()
    tok, par = host(t["node_token"]), host(t["node_parent"])
    cu = (np.arange(R + 1) * (N + 1)).astype(np.int32)
    tb = c["target"].reshape(R * (N + 1), V)
    print(f"tree verify (pctree workload) R={R} N={N} V={V}", flush=True)
    g = dsp.verify_rejection(to_gpu_bf16(tb), to_gpu(cu), t["node_token"], parent=t["node_parent"], temperature=0.0)
    torch.cuda.synchronize()
    o = ov.verify_tree_greedy(workloads.bf16_bits_to_f32(tb), cu, tok, par)
    np.testing.assert_array_equal(host(g["accepted_len"]), o["accepted_len"])
    np.testing.assert_array_equal(host(g["out_tokens"]), o["out_tokens"])
    np.testing.assert_array_equal(host(g["stop_pos"]), o["stop_node"])
    # planted paths: boost the row of each node on a random root-to-node path at its child's token
    tgt32 = workloads.bf16_bits_to_f32(c["target"]).copy()
    rng = np.random.Generator(np.random.PCG64(6))
    planted = np.zeros(R, dtype=np.int64)
    for i in range(R):
        depth = int(rng.integers(0, 17))
        cur = -1
        while planted[i] < depth:
            kids = np.flatnonzero(par[i] == cur)
            if kids.size == 0:
                break
            j = int(kids[rng.integers(0, kids.size)])
            tgt32[i, 1 + cur, tok[i, j]] = 60.0
            cur = j
            planted[i] += 1
    tb = workloads.f32_to_bf16_bits(tgt32).reshape(R * (N + 1), V)
    g = dsp.verify_rejection(to_gpu_bf16(tb), to_gpu(cu), t["node_token"], parent=t["node_parent"], temperature=0.0)
    torch.cuda.synchronize()
    o = ov.verify_tree_greedy(workloads.bf16_bits_to_f32(tb), cu, tok, par)
    np.testing.assert_array_equal(host(g["accepted_len"]), o["accepted_len"])
    np.testing.assert_array_equal(host(g["out_tokens"]), o["out_tokens"])
    np.testing.assert_array_equal(host(g["stop_pos"]), o["stop_node"])
    assert np.all(o["accepted_len"] >= planted)
    print("planted mean depth", planted.mean(), "accepted mean", o["accepted_len"].mean())


@pytest.mark.parametrize("R,depth,bits", [(5, 0, 0x7F80), (40, 0, 0x7F80), (5, 2, 0x7FC0), (40, 0, 0x7FC0),
                                          (5, 0, 0xFFC1)])
def test_tree_nonfinite_base_logit_is_a_fault(R, depth, bits):
    """A +inf or NaN base logit in request 0's row at one depth sets the non-finite status bit
    on both of the GEMM's paths (blocks of at most 16 requests add the base logits through
    the matrix cores: R = 5, and 16 parents per request at depth 3; R = 40 at depth 1 runs
    per row). Every other request still matches the oracle."""
    c = workloads.markov_case(R, 3, 3001, rank=64, seed=200 + R + depth + bits)
    L = c["L"].copy()
    L[0, depth, 17] = bits
    c = dict(c, L=L)
    _check_tree(c, 4, 16, 24, requests=range(1, R), status=dsp.DSP_STATUS_NONFINITE)


@pytest.mark.parametrize("R,D,V,rank,k,F,N,mask,bits", [
    (128, 5, 151936, 256, 4, 16, 64, False, 0),  # the PCTree shape (shorter), full row blocks
    (37, 4, 40001, 256, 4, 16, 40, True, 0),     # partial row blocks, ragged vocabulary, masked entries
    (9, 4, 5003, 64, 4, 16, 30, False, 0x7F80),  # rank 64, a +inf base logit (fault)
    (21, 3, 3001, 32, 3, 12, 20, True, 0),       # rank 32, 12 parents per request
    (16, 4, 20000, 128, 4, 16, 40, False, 0),    # rank 128
])
def test_tree_scheduled_gemm_matches_general_gemm(R, D, V, rank, k, F, N, mask, bits):
    """The tree's depths whose row blocks span at most 16 requests run on the GEMM with
    direct-to-LDS stages and a fixed issue order; it sums the same products in the same
    order as the general GEMM, so every output (tokens, parents, depths, scores, masks,
    status) must be bit-identical to a run with that kernel switched off."""
    c = workloads.markov_case(R, D, V, rank=rank, seed=300 + R + V)
    L = c["L"].copy()
    if mask:
        rng = np.random.default_rng(R)
        L[..., rng.random(V) < 0.1] = 0xFF80
    if bits:
        L[0, D - 1, 17] = bits
    c = dict(c, L=L)
    Lg, Ug, Wtg, ag = _gpu_inputs(c)
    out = {}
    try:
        for opt_on in (0, 1):
            dsp.set_option("tree_split", opt_on)
            print(f"tree R={R} D={D} V={V} rank={rank} tree_split={opt_on}", flush=True)
            g = dsp.tree_expand(Lg, Ug, Wtg, ag, k, F, N, want_mask=True)
            torch.cuda.synchronize()
            out[opt_on] = {n: host(t).copy() for n, t in g.items() if torch.is_tensor(t)}
    finally:
        dsp.set_option("tree_split", 1)
    assert (out[1]["status"][0] != 0) == bool(bits)
    for n in out[0]:
        np.testing.assert_array_equal(out[1][n].view(np.uint8), out[0][n].view(np.uint8), err_msg=n)


@pytest.mark.parametrize("R,B,V,rank,mask", [
    (256, 4, 151936, 256, False),  # the chain workload's shape (fewer steps)
    (37, 3, 40001, 256, True),     # a partial row block, ragged vocabulary, masked entries
    (300, 3, 5003, 64, False),     # two row blocks, rank 64
    (21, 3, 3001, 32, True),       # rank 32
    (16, 4, 20000, 128, False),    # rank 128
])
def test_chain_scheduled_gemm_matches_general_gemm(R, B, V, rank, mask):
    """With the opt-in scheduled GEMM, the greedy chain's arg-max steps (no log q) run on the
    kernel with direct-to-LDS stages and a fixed issue order; it starts the accumulators
    from L and sums the k-steps in the same order as the general GEMM, so the tokens must be
    identical to the general kernel's, and to the oracle up to counted near-ties."""
    c = workloads.markov_case(R, B, V, rank=rank, seed=400 + R + V)
    if mask:
        L = c["L"].copy()
        L[..., np.random.default_rng(R).random(V) < 0.1] = 0xFF80
        c = dict(c, L=L)
    Lg, Ug, Wtg, ag = _gpu_inputs(c)
    out = {}
    try:
        for opt_on in (0, 1):
            dsp.set_option("chain_sched", opt_on)
            print(f"chain R={R} B={B} V={V} rank={rank} chain_sched={opt_on}", flush=True)
            g = dsp.draft_markov_step(Lg, Ug, Wtg, ag)
            torch.cuda.synchronize()
            assert int(host(g["status"])[0]) == 0
            out[opt_on] = host(g["y"]).copy()
        dsp.set_option("chain_sched", 1)
        _check_chain(c, want_logq=False, requests=range(0, R, max(1, R // 24)))
    finally:
        dsp.set_option("chain_sched", 0)
    np.testing.assert_array_equal(out[1], out[0])
