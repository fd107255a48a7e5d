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
