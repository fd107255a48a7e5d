"""Pins of the oracle's verify step against what the pages and the mathematics fix.

DSpark study notes, section 1: rejection sampling keeps the target distribution
exactly; section 3 / Figure 1: a rejected draft is replaced by the target's own
token. DSpark notes section 5.1: the one-token acceptance rate is
sum_v min(p_v, q_v) = 1 - TV(p, q). PCTree article: greedy decoding checks that
drafts match the target's choice.
"""
import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import verify as ov

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _packed(t):
    """Dense [R, K+1, V] target with full windows -> packed rows and cu_seqlens."""
    R, K1, V = t.shape
    return t.reshape(R * K1, V), np.arange(R + 1, dtype=np.int32) * K1


def test_greedy_equals_argmax_prefix_matching():
    rng = np.random.Generator(np.random.PCG64(11))
    R, K, V = 40, 6, 37
    t = rng.standard_normal((R, K + 1, V))
    am = np.argmax(t, axis=-1)
    # plant the target's argmax for a random number of leading positions, then a miss
    x = rng.integers(0, V, size=(R, K))
    lead = rng.integers(0, K + 1, size=R)
    for i in range(R):
        x[i, :lead[i]] = am[i, :lead[i]]
        if lead[i] < K and x[i, lead[i]] == am[i, lead[i]]:
            x[i, lead[i]] = (am[i, lead[i]] + 1) % V
    tp, cu = _packed(t)
    res = ov.verify_chain(tp, cu, np.zeros((R, K, V)), x, temperature=0.0)
    np.testing.assert_array_equal(res["accepted_len"], lead)
    for i in range(R):
        n = lead[i]
        np.testing.assert_array_equal(res["out_tokens"][i, :n], am[i, :n])
        assert res["out_tokens"][i, n] == am[i, n]  # target's own token at the stop
        assert np.all(res["out_tokens"][i, n + 1:] == -1)


def test_greedy_ties_take_lowest_token():
    t = np.zeros((1, 2, 5))
    t[0, 0, [1, 3]] = 2.0
    t[0, 1, [0, 4]] = -0.0
    t[0, 1, 2] = -1.0
    tp, cu = _packed(t)
    res = ov.verify_chain(tp, cu, np.zeros((1, 1, 5)), np.array([[3]]), temperature=0.0)
    assert res["accepted_len"][0] == 0 and res["out_tokens"][0, 0] == 1
    res = ov.verify_chain(tp, cu, np.zeros((1, 1, 5)), np.array([[1]]), temperature=0.0)
    assert res["accepted_len"][0] == 1 and res["out_tokens"][0, 1] == 0


def test_identical_draft_accepts_whole_block():
    rng = np.random.Generator(np.random.PCG64(12))
    R, K, V = 30, 7, 50
    t = rng.standard_normal((R, K + 1, V)) * 2
    d = t[:, :K].copy()
    x = rng.integers(0, V, size=(R, K))
    tp, cu = _packed(t)
    for T in (1.0, 0.7):
        res = ov.verify_chain(tp, cu, d, x, temperature=T, seed=5, rnd=1)
        np.testing.assert_array_equal(res["accepted_len"], K)
        np.testing.assert_array_equal(res["out_tokens"][:, :K], x)
        np.testing.assert_allclose(res["p_x"], res["q_x"], rtol=0, atol=0)


def _two_token_case(a, R, K, seed):
    """V = 2 rows with p = (a/2, 1-a/2), q = (1-a/2, a/2): acceptance exactly a per position."""
    p = np.array([a / 2, 1 - a / 2])
    q = np.array([1 - a / 2, a / 2])
    t = np.broadcast_to(np.log(p), (R, K + 1, 2)).copy()
    d = np.broadcast_to(np.log(q), (R, K, 2)).copy()
    x = (np.random.Generator(np.random.PCG64(seed)).random((R, K)) >= q[0]).astype(np.int64)
    return t, d, x


@pytest.mark.parametrize("a,K", [(0.3, 1), (0.6, 7), (0.9, 16), (0.6, 1), (0.9, 7)])
def test_expected_accepted_length_closed_form(a, K):
    R = 6000
    t, d, x = _two_token_case(a, R, K, seed=int(a * 100) + K)
    tp, cu = _packed(t)
    res = ov.verify_chain(tp, cu, d, x, temperature=1.0, seed=0, rnd=K)
    tau = res["accepted_len"] + 1.0  # acceptance length counts the bonus / corrected token
    expect = (1 - a ** (K + 1)) / (1 - a)
    se = tau.std(ddof=1) / np.sqrt(R)
    assert abs(tau.mean() - expect) < 5 * se + 1e-12, (tau.mean(), expect, se)


def _vocab8_case(R, K, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    t_rows = rng.standard_normal((K + 1, 8)) * 1.5
    d_rows = t_rows[:K] + rng.standard_normal((K, 8)) * 0.8
    t = np.broadcast_to(t_rows, (R, K + 1, 8)).copy()
    d = np.broadcast_to(d_rows, (R, K, 8)).copy()
    q = np.exp(d_rows - d_rows.max(1, keepdims=True))
    q /= q.sum(1, keepdims=True)
    x = np.stack([rng.choice(8, size=R, p=q[k]) for k in range(K)], axis=1)
    p = np.exp(t_rows - t_rows.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    return t, d, x, p, q


def test_vocab8_exact_enumeration_first_token_law():
    """Enumerate x_1 under q_1: the law of the first committed token equals p_1 to 1e-12.

    The accept branch has probability min(1, ratio) over u ~ U[0, 1), with the
    ratio exp(lp - lq) built from the oracle's own log-softmax; the reject
    branch commits the oracle's inverse-CDF draw from the residual, whose law
    over u' is integrated by probing the sampler inside every CDF interval.
    """
    t, d, _, _, _ = _vocab8_case(1, 2, seed=21)
    lp = ov.log_softmax(t[0, 0], 1.0)
    lq = ov.log_softmax(d[0, 0], 1.0)
    p, q = np.exp(lp), np.exp(lq)
    law = np.zeros(8)
    for x1 in range(8):
        acc = min(1.0, float(np.exp(lp[x1] - lq[x1])))
        law[x1] += q[x1] * acc
        r = np.maximum(0.0, p - q)
        edges = np.concatenate([[0.0], np.cumsum(r) / r.sum()])
        for v in range(8):
            lo, hi = edges[v], edges[v + 1]
            if hi > lo:
                assert ov.inverse_cdf(r, 0.5 * (lo + hi))[0] == v
                law[v] += q[x1] * (1 - acc) * (hi - lo)
    np.testing.assert_allclose(law, p, rtol=0, atol=1e-12)


def test_vocab8_monte_carlo_target_law():
    R, K = 30000, 2
    t, d, x, p, q = _vocab8_case(R, K, seed=22)
    tp, cu = _packed(t)
    res = ov.verify_chain(tp, cu, d, x, temperature=1.0, seed=3, rnd=0)
    first = res["out_tokens"][:, 0]
    chi2, pv = stats.chisquare(np.bincount(first, minlength=8), R * p[0])
    assert pv > 1e-3, (chi2, pv)
    # given the first draft was accepted, position 2 is a fresh verify: committed token ~ p_2
    sel = res["accepted_len"] >= 1
    second = res["out_tokens"][sel, 1]
    chi2, pv = stats.chisquare(np.bincount(second, minlength=8), sel.sum() * p[1])
    assert pv > 1e-3, (chi2, pv)
    # with the whole block accepted the bonus is drawn from p_{K+1}
    sel = res["accepted_len"] == K
    bonus = res["out_tokens"][sel, K]
    chi2, pv = stats.chisquare(np.bincount(bonus, minlength=8), sel.sum() * p[K])
    assert pv > 1e-3, (chi2, pv)
    # position-1 acceptance rate = sum_v min(p_v, q_v) = 1 - TV
    rate = (res["accepted_len"] >= 1).mean()
    a = np.minimum(p[0], q[0]).sum()
    assert abs(rate - a) < 5 * np.sqrt(a * (1 - a) / R)


def test_reported_probabilities():
    R, K = 3, 2
    t, d, x, p, q = _vocab8_case(R, K, seed=23)
    tp, cu = _packed(t)
    res = ov.verify_chain(tp, cu, d, x, temperature=1.0)
    for i in range(R):
        for k in range(K):
            np.testing.assert_allclose(res["p_x"][i, k], p[k, x[i, k]], rtol=1e-13)
            np.testing.assert_allclose(res["q_x"][i, k], q[k, x[i, k]], rtol=1e-13)


def test_temperature_scales_logits():
    # softmax(t / T) at T = 2 equals softmax of the halved logits at T = 1
    R, K = 200, 3
    t, d, x, p, q = _vocab8_case(R, K, seed=24)
    tp, cu = _packed(t)
    a = ov.verify_chain(tp, cu, d, x, temperature=2.0, seed=1)
    b = ov.verify_chain(tp / 2, cu, d / 2, x, temperature=1.0, seed=1)
    np.testing.assert_array_equal(a["accepted_len"], b["accepted_len"])
    np.testing.assert_array_equal(a["out_tokens"], b["out_tokens"])


def test_ragged_windows_and_zero_window():
    rng = np.random.Generator(np.random.PCG64(25))
    K, V = 4, 16
    win = np.array([0, 4, 2, 1])
    R = len(win)
    rows = [rng.standard_normal((n + 1, V)) for n in win]
    tp = np.concatenate(rows)
    cu = np.concatenate([[0], np.cumsum(win + 1)]).astype(np.int32)
    d = rng.standard_normal((R, K, V))
    x = rng.integers(0, V, size=(R, K))
    res = ov.verify_chain(tp, cu, d, x, temperature=0.0)
    assert res["accepted_len"][0] == 0 and res["out_tokens"][0, 0] == np.argmax(rows[0][0])
    assert np.all(res["accepted_len"] <= win)
    res = ov.verify_chain(tp, cu, d, x, temperature=1.0)
    assert np.all(res["accepted_len"] <= win)
    assert np.all(res["p_x"][0] == 0) and np.all(res["p_x"][3, 1:] == 0)


def test_figure1_cycle_greedy():
    g = json.load(open(os.path.join(GOLD, "figure1_cycle.json")))
    tok = g["tokens"]
    V = g["vocab"]
    win = g["expected_window"]
    drafts = [tok[s] for s in g["drafts"]]
    rows = []
    ctx = [g["anchor"]] + g["drafts"][:win]
    for s in ctx:
        r = np.zeros(V)
        r[tok[g["target_argmax_after"][s]]] = 5.0
        rows.append(r)
    tp = np.stack(rows)
    cu = np.array([0, win + 1], dtype=np.int32)
    res = ov.verify_chain(tp, cu, np.zeros((1, 4, V)), np.array([drafts]), temperature=0.0)
    assert res["accepted_len"][0] == g["expected_accepted"]
    assert [int(v) for v in res["out_tokens"][0, :3]] == [tok[s] for s in g["expected_committed"]]


def test_tree_walk_chain_shaped_equals_chain_greedy():
    rng = np.random.Generator(np.random.PCG64(26))
    R, K, V = 20, 5, 11
    t = rng.standard_normal((R, K + 1, V))
    am = np.argmax(t, axis=-1)
    x = np.where(rng.random((R, K)) < 0.7, am[:, :K], rng.integers(0, V, size=(R, K)))
    tp, cu = _packed(t)
    chain = ov.verify_chain(tp, cu, np.zeros((R, K, V)), x, temperature=0.0)
    parent = np.tile(np.arange(-1, K - 1), (R, 1))
    tree = ov.verify_tree_greedy(tp, cu, x, parent)
    np.testing.assert_array_equal(tree["accepted_len"], chain["accepted_len"])
    np.testing.assert_array_equal(tree["out_tokens"], chain["out_tokens"])


def test_tree_walk_planted_path():
    rng = np.random.Generator(np.random.PCG64(27))
    V, N = 30, 12
    # root has children 0,1,2; node 1 has children 3,4; node 4 has child 5; others chained
    parent = np.array([-1, -1, -1, 1, 1, 4, 0, 6, 2, 3, 5, 9])
    token = np.array([3, 7, 9, 1, 2, 5, 4, 8, 6, 11, 12, 13])
    rows = rng.standard_normal((N + 1, V))
    planted = [1, 4, 5, 10]  # root -> 1 -> 4 -> 5 -> 10
    cur = -1
    for j in planted:
        rows[1 + cur, token[j]] = 10.0
        cur = j
    rows[1 + cur] = rows[1 + cur] - 20  # make sure no child of node 10 is picked
    rows[1 + cur, 0] = 1.0
    cu = np.array([0, N + 1], dtype=np.int32)
    res = ov.verify_tree_greedy(rows, cu, token[None], parent[None])
    assert res["accepted_len"][0] == 4
    assert list(res["out_tokens"][0, :4]) == [token[j] for j in planted]
    assert res["out_tokens"][0, 4] == 0 and res["stop_node"][0] == 10


# ---- cap-accept (SGLang article, "three verify modes" and "observability")


def _cap_case(seed, R=12, K=6, V=29, T=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    t = rng.standard_normal((R, K + 1, V)) * 2.0
    d = np.concatenate([t[:, :K] + rng.standard_normal((R, K, V)) * 0.6], axis=0)
    Td = T if T > 0 else 1.0  # draft tokens drawn from softmax(d) (argmax-free at T = 0 too)
    x = np.array([[rng.choice(V, p=np.exp(ov.log_softmax(d[i, k], Td))) for k in range(K)] for i in range(R)])
    cap = rng.integers(0, K + 2, size=R)  # includes caps beyond the block
    return t, d, x, cap


@pytest.mark.parametrize("seed,T", [(1, 1.0), (2, 0.7), (3, 0.0), (4, 1.0)])
def test_cap_accept_commits_what_compact_commits(seed, T):
    """The committed result equals verifying only the window (compact): the same
    uniforms, keyed by request and position, make every committed decision and
    the draw identical; only the packing differs."""
    t, d, x, cap = _cap_case(seed, T=T)
    R, K1, V = t.shape
    K = K1 - 1
    tp, cu = _packed(t)
    full = ov.verify_chain(tp, cu, d, x, T, seed=9, rnd=3, cap=cap)
    c = np.minimum(cap, K)
    tpc = np.concatenate([t[i, :c[i] + 1] for i in range(R)])
    cuc = np.concatenate([[0], np.cumsum(c + 1)]).astype(np.int32)
    compact = ov.verify_chain(tpc, cuc, d, x, T, seed=9, rnd=3)
    for key in ("accepted_len", "out_tokens", "stop_pos"):
        np.testing.assert_array_equal(full[key], compact[key])


@pytest.mark.parametrize("seed,T", [(5, 1.0), (6, 0.0)])
def test_cap_accept_ceiling_is_the_full_block_verify(seed, T):
    t, d, x, cap = _cap_case(seed, T=T)
    tp, cu = _packed(t)
    full = ov.verify_chain(tp, cu, d, x, T, seed=2, rnd=1, cap=cap)
    static = ov.verify_chain(tp, cu, d, x, T, seed=2, rnd=1)
    np.testing.assert_array_equal(full["ceiling"], static["accepted_len"])
    np.testing.assert_array_equal(static["ceiling"], static["accepted_len"])
    assert np.all(full["accepted_len"] == np.minimum(full["ceiling"], np.minimum(cap, t.shape[1] - 1)))
    # a cap at or beyond the block is the static verify itself
    wide = ov.verify_chain(tp, cu, d, x, T, seed=2, rnd=1, cap=np.full(len(cap), 99))
    for key in ("accepted_len", "out_tokens", "stop_pos"):
        np.testing.assert_array_equal(wide[key], static[key])


def test_scheduled_tv_fixture_is_current():
    """The stored total-variation distances behind the scheduled workload's confidences match
    the oracle's fp64 softmax on sampled (request, position) pairs of the current logits."""
    import workloads
    from oracle.calibrate_scheduled_verify import tv_table
    c = workloads.scheduled_verify(R=256, K=16)
    sub = dict(c, R=3, t=c["t"][[0, 100, 255]], d=c["d"][[0, 100, 255]])
    tv = tv_table(sub)
    np.testing.assert_allclose(tv, c["tv"][[0, 100, 255]], atol=1e-6)
    assert np.all((c["tv"] >= 0) & (c["tv"] <= 1))
