"""Pins of the oracle's PCTree expansion (PCTree article)."""
import itertools
import math

import numpy as np
import pytest

import workloads
from oracle import markov as om
from oracle import pctree as opt


def _case(R, D, V, r=32, seed=1, boost=1.0):
    c = workloads.markov_case(R, D, V, rank=r, seed=seed)
    L = workloads.bf16_bits_to_f32(c["L"])
    U = workloads.bf16_bits_to_f32(c["U"])
    W = workloads.bf16_bits_to_f32(c["W"]) * np.float32(boost)
    return L, U, W, c["anchors"]


def test_k1_f1_reduces_to_chain():
    L, U, W, a = _case(4, 6, 120, seed=2, boost=300)
    tree = opt.tree_expand(L, U, W, a, topk=1, frontier=1, topN=6)
    chain = om.chain(L, U, W, a)
    np.testing.assert_array_equal(tree["node_token"], chain["y"])
    np.testing.assert_array_equal(tree["node_parent"], np.tile(np.arange(-1, 5), (4, 1)))
    np.testing.assert_array_equal(tree["node_depth"], np.tile(np.arange(1, 7), (4, 1)))
    np.testing.assert_allclose(tree["node_score"], np.cumsum(chain["logq"], axis=1), rtol=1e-12)


def _lse(z):
    m = max(z)
    return m + math.log(math.fsum(math.exp(v - m) for v in z))


def test_no_pruning_equals_brute_force_over_all_paths():
    """Tiny vocabulary, k = V and F >= V^(D-1): top-N of every path by summed log-probability."""
    V, D, N = 4, 3, 20
    L, U, W, a = _case(1, D, V, r=32, seed=5, boost=600)
    L64, U64, W64 = L[0].astype(np.float64), U.astype(np.float64), W.astype(np.float64)
    paths = []
    for depth in range(1, D + 1):
        for toks in itertools.product(range(V), repeat=depth):
            prev, s = int(a[0]), 0.0
            for d, v in enumerate(toks):
                z = [float(L64[d, w]) + math.fsum(U64[prev, j] * W64[j, w] for j in range(32))
                     for w in range(V)]
                s += z[v] - _lse(z)
                prev = v
            paths.append((s, depth, toks))
    paths.sort(key=lambda p: (-p[0], p[1]))
    tree = opt.tree_expand(L, U, W, a, topk=V, frontier=V ** (D - 1), topN=N)
    assert tree["n_nodes"][0] == N
    got = []
    for j in range(N):
        toks, cur = [], j
        while cur >= 0:
            toks.append(int(tree["node_token"][0, cur]))
            cur = int(tree["node_parent"][0, cur])
        got.append(tuple(reversed(toks)))
    assert got == [p[2] for p in paths[:N]]
    np.testing.assert_allclose(tree["node_score"][0], [p[0] for p in paths[:N]], rtol=1e-10)


@pytest.mark.parametrize("k,F,N", [(4, 16, 64), (3, 5, 12), (2, 7, 40)])
def test_tree_invariants(k, F, N):
    R, D, V = 3, 8, 500
    L, U, W, a = _case(R, D, V, seed=7, boost=200)
    t = opt.tree_expand(L, U, W, a, topk=k, frontier=F, topN=N)
    for i in range(R):
        n = t["n_nodes"][i]
        f, kept = 1, 0
        for _ in range(D):
            f = min(F, k * f)
            kept += f
        assert n == min(N, kept)
        par, tok, dep, sc = (t["node_parent"][i, :n], t["node_token"][i, :n],
                             t["node_depth"][i, :n], t["node_score"][i, :n])
        for j in range(n):
            assert par[j] < j
            if par[j] >= 0:
                assert dep[par[j]] == dep[j] - 1 and sc[par[j]] >= sc[j]
            else:
                assert dep[j] == 1
        assert np.all(np.diff(sc) <= 0)
        for p in set(par.tolist()):
            sib = tok[par == p]
            assert len(set(sib.tolist())) == len(sib)
        for d in range(1, D + 1):
            assert (dep == d).sum() <= F


def test_ancestor_masks_chain_closed_form():
    """A chain-shaped tree: node j's ancestors-or-self are 0..j, i.e. the low j+1 bits."""
    N = 130
    par = np.arange(-1, N - 1)[None]
    m = opt.ancestor_masks(par, [N])
    for j in range(N):
        want = [0, 0, 0]
        for a in range(j + 1):
            want[a // 64] |= 1 << (a % 64)
        assert [int(x) for x in m[0, j]] == want


def test_ancestor_masks_popcount_is_depth_and_closed():
    L, U, W, a = _case(3, 4, 200, seed=6, boost=200)
    t = opt.tree_expand(L, U, W, a, topk=3, frontier=5, topN=12)
    m = opt.ancestor_masks(t["node_parent"], t["n_nodes"])
    for i in range(3):
        for j in range(int(t["n_nodes"][i])):
            bits = [b for b in range(12) if (int(m[i, j, 0]) >> b) & 1]
            assert len(bits) == t["node_depth"][i, j]
            assert j in bits and max(bits) == j
            p = t["node_parent"][i, j]
            if p >= 0:
                assert int(m[i, j, 0]) == int(m[i, p, 0]) | (1 << j)
        assert np.all(m[i, int(t["n_nodes"][i]):] == 0)


def _as_prefer(t):
    return t["node_token"], t["node_parent"], t["n_nodes"]


def test_replay_of_own_tree_changes_nothing():
    L, U, W, a = _case(3, 6, 400, seed=11, boost=200)
    own = opt.tree_expand(L, U, W, a, 4, 8, 24)
    rep = opt.tree_expand(L, U, W, a, 4, 8, 24, prefer=_as_prefer(own))
    for k in ("node_token", "node_parent", "node_depth", "n_nodes"):
        np.testing.assert_array_equal(rep[k], own[k])
    np.testing.assert_array_equal(rep["node_score"], own["node_score"])
    assert np.all(rep["replays"] == 0)
    assert np.all(rep["decisions"] > 6)


def _planted_topk_tie(delta):
    """One request, depth 3, no Markov term: at depth 1 tokens 5 and 9 sit at the top-2 cut
    (k = 2) with z differing by delta; token 5 ranks first at every depth otherwise."""
    V, D = 64, 3
    rng = np.random.default_rng(3)
    L = rng.normal(0.0, 1.0, (1, D, V))
    L[0, 0, 1] = 4.0
    L[0, 0, 5] = 3.0 + delta
    L[0, 0, 9] = 3.0
    U, W = np.zeros((V, 32)), np.zeros((32, V))
    return L, U, W, np.array([0])


def test_replay_takes_the_other_branch_at_a_planted_near_tie():
    """The oracle keeps token 5 (z larger by 1e-9); a tree built with token 9 instead (the
    rounding could have gone either way) is reproduced exactly by the replay, one near-tie."""
    L, U, W, a = _planted_topk_tie(1e-9)
    own = opt.tree_expand(L, U, W, a, 2, 4, 12)
    assert 5 in own["node_token"][0, own["node_depth"][0] == 1]
    L2 = L.copy()
    L2[0, 0, 5] = 3.0 - 1e-9
    other = opt.tree_expand(L2, U, W, a, 2, 4, 12)
    assert 9 in other["node_token"][0, other["node_depth"][0] == 1]
    rep = opt.tree_expand(L, U, W, a, 2, 4, 12, prefer=_as_prefer(other))
    for k in ("node_token", "node_parent", "node_depth", "n_nodes"):
        np.testing.assert_array_equal(rep[k], other[k])
    np.testing.assert_allclose(rep["node_score"], other["node_score"], atol=1e-8)
    assert rep["replays"][0] >= 1


def test_replay_refuses_a_branch_outside_the_band():
    """The same plant with a gap of 1e-3: the other tree's choice is no near-tie, so the
    replay keeps the oracle's own tree (a checker comparing against it then fails)."""
    L, U, W, a = _planted_topk_tie(1e-3)
    own = opt.tree_expand(L, U, W, a, 2, 4, 12)
    L2 = L.copy()
    L2[0, 0, 5] = 3.0 - 1e-3
    other = opt.tree_expand(L2, U, W, a, 2, 4, 12)
    assert not np.array_equal(own["node_token"], other["node_token"])
    rep = opt.tree_expand(L, U, W, a, 2, 4, 12, prefer=_as_prefer(other))
    np.testing.assert_array_equal(rep["node_token"], own["node_token"])
    assert rep["replays"][0] == 0


def test_replay_at_a_planted_frontier_near_tie():
    """k = 3, F = 2: at depth 1 the 2nd and 3rd children's path scores differ by 1e-10 only;
    the replay follows whichever of the two the preferred tree kept."""
    V, D = 50, 3
    rng = np.random.default_rng(8)
    L = rng.normal(0.0, 1.0, (1, D, V))
    L[0, 0, 2] = 5.0
    L[0, 0, 7] = 4.0 + 1e-10
    L[0, 0, 30] = 4.0
    U, W = np.zeros((V, 32)), np.zeros((32, V))
    a = np.array([0])
    own = opt.tree_expand(L, U, W, a, 3, 2, 6)
    d1 = set(own["node_token"][0, own["node_depth"][0] == 1].tolist())
    assert d1 == {2, 7}
    L2 = L.copy()
    L2[0, 0, 7] = 4.0 - 1e-10
    other = opt.tree_expand(L2, U, W, a, 3, 2, 6)
    assert set(other["node_token"][0, other["node_depth"][0] == 1].tolist()) == {2, 30}
    rep = opt.tree_expand(L, U, W, a, 3, 2, 6, prefer=_as_prefer(other))
    for k in ("node_token", "node_parent", "node_depth"):
        np.testing.assert_array_equal(rep[k], other[k])
    assert rep["replays"][0] >= 1


def test_topk_decides_on_fp64_values():
    """Two tokens equal in fp32 but not in fp64 at the top-1 cut: the larger fp64 value wins."""
    z = np.zeros(10)
    z[3] = 1.0
    z[8] = 1.0 + 2.0 ** -40
    top, gap, _ = opt._topk_tokens(z, 1)
    assert list(top) == [8] and abs(gap - 2.0 ** -40) < 2.0 ** -70
    z[8] = 1.0
    top, _, _ = opt._topk_tokens(z, 1)
    assert list(top) == [3]
