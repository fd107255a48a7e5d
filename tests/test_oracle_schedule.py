"""Pins of the oracle's survival products and prefix scheduler.

DSpark study notes, section 5.1-5.2: survival is the running product of the
confidences; throughput = expected accepted tokens x steps-per-second at the
batch size; the greedy order by survival is optimal because the marginal gain
of extending a request to position k is S_{i,k}; the early stop keeps every
decision dependent on the prefix only. SGLang article: additive step-time table.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import schedule as osch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _brute_force_best_J(conf, a, b):
    """max over every window vector n in {0..K}^R of E(n) / c(sum n), unquantised fp64."""
    conf = np.asarray(conf, dtype=np.float64)
    R, K = conf.shape
    S = np.cumprod(conf, axis=1)
    best = 0.0 / a
    for n in itertools.product(range(K + 1), repeat=R):
        E = sum(S[i, :n[i]].sum() for i in range(R))
        best = max(best, E / (a + b * sum(n)))
    return best


@pytest.mark.parametrize("seed", range(12))
def test_matches_brute_force_optimum(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    R, K = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    conf = rng.uniform(0.05, 1.0, size=(R, K)).astype(np.float32)
    a, b = float(rng.uniform(0.2, 2.0)), float(rng.uniform(0.0, 0.6))
    cost = osch.additive_cost(a, b, R * K)
    best = _brute_force_best_J(conf, a, b)
    for mode in (osch.MODE_EARLY_STOP, osch.MODE_ARGMAX):
        r = osch.schedule_windows(conf, cost, mode=mode)
        S = np.cumprod(conf.astype(np.float64), axis=1)
        E = sum(S[i, :r["windows"][i]].sum() for i in range(R))
        J = E / cost[r["windows"].sum()]
        assert J >= best * (1 - 1e-9), (mode, J, best)
        assert r["N"] == r["windows"].sum()


def test_early_stop_equals_argmax_for_additive_tables():
    rng = np.random.Generator(np.random.PCG64(99))
    for _ in range(30):
        R, K = int(rng.integers(1, 40)), int(rng.integers(1, 17))
        conf = rng.uniform(0.0, 1.0, size=(R, K)).astype(np.float32)
        cost = osch.additive_cost(float(rng.uniform(0.1, 3)), float(rng.uniform(0, 0.3)), R * K)
        e = osch.schedule_windows(conf, cost, osch.MODE_EARLY_STOP)["windows"]
        g = osch.schedule_windows(conf, cost, osch.MODE_ARGMAX)["windows"]
        np.testing.assert_array_equal(e, g)


def test_survival_products():
    conf = np.array([[0.5, 0.5, 0.5, 1.0], [1.0, 0.25, 0.0, 0.9]], dtype=np.float32)
    S = osch.survival(conf)
    np.testing.assert_array_equal(S[0], [0.5, 0.25, 0.125, 0.125])
    np.testing.assert_array_equal(S[1], [1.0, 0.25, 0.0, 0.0])
    rng = np.random.Generator(np.random.PCG64(3))
    S = osch.survival(rng.uniform(0, 1, size=(50, 16)).astype(np.float32))
    assert np.all(np.diff(S, axis=1) <= 0)


def test_special_cases():
    R, K = 5, 6
    ones = np.ones((R, K), np.float32)
    zeros = np.zeros((R, K), np.float32)
    cost = osch.additive_cost(1.0, 0.05, R * K)
    np.testing.assert_array_equal(osch.schedule_windows(ones, cost)["windows"], K)
    np.testing.assert_array_equal(osch.schedule_windows(zeros, cost)["windows"], 0)
    # flat table: every candidate with nonzero survival raises throughput
    conf = np.random.Generator(np.random.PCG64(4)).uniform(0.01, 1, size=(R, K)).astype(np.float32)
    conf[2, 3] = 0.0
    w = osch.schedule_windows(conf, np.ones(R * K + 1))["windows"]
    expect = np.full(R, K)
    expect[2] = 3
    np.testing.assert_array_equal(w, expect)
    # zero step time everywhere: no candidate strictly raises E / c, nothing is verified
    np.testing.assert_array_equal(osch.schedule_windows(conf, np.zeros(R * K + 1))["windows"], 0)


def test_non_anticipation():
    """Lowering the confidence of candidates ranked after the stop leaves the windows unchanged."""
    rng = np.random.Generator(np.random.PCG64(5))
    for _ in range(20):
        R, K = 8, 10
        conf = rng.uniform(0.3, 1.0, size=(R, K)).astype(np.float32)
        cost = osch.additive_cost(1.0, 0.08, R * K)
        w = osch.schedule_windows(conf, cost)["windows"]
        assert 0 < w.sum() < R * K
        low = conf.copy()
        for i in range(R):
            if w[i] < K:
                low[i, w[i]:] *= rng.uniform(0.0, 1.0, size=K - w[i]).astype(np.float32)
        np.testing.assert_array_equal(osch.schedule_windows(low, cost)["windows"], w)


def test_prefix_closed_order():
    rng = np.random.Generator(np.random.PCG64(6))
    conf = rng.uniform(0.0, 1.0, size=(30, 12)).astype(np.float32)
    conf[:, 5] = 1.0  # equal survivals inside a request: ties keep position order
    r = osch.schedule_windows(conf, osch.additive_cost(1, 0.01, 360))
    ci, ck = r["order"]
    for i in range(30):
        ks = ck[ci == i]
        np.testing.assert_array_equal(ks, np.arange(12))


def test_higher_step_cost_never_verifies_more():
    rng = np.random.Generator(np.random.PCG64(7))
    conf = rng.uniform(0.2, 1.0, size=(32, 16)).astype(np.float32)
    Ns = [osch.schedule_windows(conf, osch.additive_cost(1.0, b, 512))["N"]
          for b in (0.0, 0.01, 0.02, 0.05, 0.1, 0.3, 1.0)]
    assert all(x >= y for x, y in zip(Ns, Ns[1:])), Ns
    assert Ns[0] == 512


def test_capacity_cap():
    conf = np.full((4, 8), 0.99, np.float32)
    r = osch.schedule_windows(conf, np.ones(33), max_tokens=10)
    assert r["N"] == 10 and r["windows"].sum() == 10


def test_quantisation_keeps_sums_exact():
    for R, K in [(1, 1), (256, 16), (512, 16), (4096, 16), (8192, 64)]:
        Q = osch.quant_bits(R, K)
        assert R * K * 2 ** Q <= 2 ** 53
    assert osch.quant_bits(256, 16) == 40


def test_figure1_window():
    g = json.load(open(os.path.join(GOLD, "figure1_cycle.json")))
    conf = np.array([g["confidence"]], dtype=np.float32)
    cost = osch.additive_cost(g["cost_a"], g["cost_b"], 4)
    for mode in (osch.MODE_EARLY_STOP, osch.MODE_ARGMAX):
        assert osch.schedule_windows(conf, cost, mode)["windows"][0] == g["expected_window"]


# ---- scheduler variants: fixed capacity from an older step (top-M) and fixed threshold


def test_threshold_zero_is_full_block():
    """Notes 8.3, Figure 5: threshold 0 is the conventional verify-everything block."""
    rng = np.random.default_rng(3)
    conf = rng.uniform(0.0, 1.0, size=(9, 7)).astype(np.float32)
    r = osch.schedule_windows(conf, np.ones(64), mode=osch.MODE_THRESHOLD, threshold=0.0)
    assert np.array_equal(r["windows"], np.full(9, 7))
    assert r["N"] == 63


def test_threshold_hand_case():
    # survivals (float32 confidences multiplied in fp64): row 0: 0.9, 0.72, 0.36; row 1: 0.5, 0.45, 0.405
    conf = np.array([[0.9, 0.8, 0.5], [0.5, 0.9, 0.9]], np.float32)
    cost = np.ones(7)
    for th, want in [(0.3, [3, 3]), (0.4, [2, 3]), (0.42, [2, 2]), (0.46, [2, 1]), (0.6, [2, 0]), (0.8, [1, 0]),
                     (0.95, [0, 0])]:
        r = osch.schedule_windows(conf, cost, mode=osch.MODE_THRESHOLD, threshold=th)
        assert r["windows"].tolist() == want, th
        assert r["N"] == sum(want)


def test_threshold_monotone_and_prefix():
    rng = np.random.default_rng(4)
    conf = rng.uniform(0.3, 1.0, size=(20, 9)).astype(np.float32)
    prev = None
    for th in np.linspace(0.0, 1.0, 21):
        w = osch.schedule_windows(conf, np.ones(181), mode=osch.MODE_THRESHOLD, threshold=th)["windows"]
        S = np.cumprod(conf.astype(np.float64), axis=1)
        assert np.array_equal(w, (S >= th).sum(axis=1))  # S is non-increasing, so a prefix
        if prev is not None:
            assert np.all(w <= prev)
        prev = w


def _exact_order(conf):
    """Candidates by exact fp64 survival descending, ties by request then position."""
    S = np.cumprod(conf.astype(np.float64), axis=1)
    R, K = S.shape
    return sorted(((i, k) for i in range(R) for k in range(K)), key=lambda t: (-S[t], t[0], t[1]))


def test_top_m_takes_the_m_best_candidates():
    rng = np.random.default_rng(5)
    conf = rng.uniform(0.2, 1.0, size=(11, 6)).astype(np.float32)
    order = _exact_order(conf)
    for M in (0, 1, 7, 30, 65, 66):
        r = osch.schedule_windows(conf, np.ones(67), mode=osch.MODE_TOP_M, max_tokens=M)
        want = np.zeros(11, np.int32)
        for i, _ in order[:M]:
            want[i] += 1
        assert np.array_equal(r["windows"], want), M
        assert r["N"] == M


def test_top_m_at_the_early_stop_capacity_reproduces_it():
    """With the capacity the early stop would choose, the ranking from the same
    survivals gives the same windows (the async rule only delays the capacity)."""
    rng = np.random.default_rng(6)
    conf = rng.uniform(0.1, 1.0, size=(16, 8)).astype(np.float32)
    cost = osch.additive_cost(1.0, 0.05, 128)
    es = osch.schedule_windows(conf, cost)
    tm = osch.schedule_windows(conf, cost, mode=osch.MODE_TOP_M, max_tokens=es["N"])
    assert np.array_equal(es["windows"], tm["windows"])
    small = osch.schedule_windows(conf, cost, mode=osch.MODE_TOP_M, max_tokens=es["N"] // 2)
    assert np.all(small["windows"] <= es["windows"])
