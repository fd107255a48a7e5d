"""Parent-conditioned drafting tree (PCTree) expansion -- oracle side (test infrastructure).

Follows the PCTree article (qiita.com, "a straight draft wastes everything
after the first miss"): the Markov head is a function that scores the children
of one given parent token, so for every parent p on the current frontier the
expansion computes z_d(p) = L_d + Markov(p) (all frontier parents in one batched
Markov call), keeps a local top-k of children per parent, ranks every path by
its summed log-probability s(c) = sum log pi(v | u), prunes each depth to a
top-k frontier, and finally keeps a global top-N of the nodes that fits the
verify budget; one target forward then verifies the whole tree. No extra
backbone pass and no retraining are needed.

Per request, with the root = the anchor token and score 0:
  for depth d = 1..D, for each parent p in frontier F_{d-1} (in slot order):
      z = L_{i,d} + U[tok(p)] @ W  (fp64),  lse = logsumexp(z)
      children = top-k tokens of z by (z desc, token asc), z rounded to fp32 for the decision
      child score s = s(p) + (z_v - lse)            (fp64, log pi = z_v - lse)
  F_d = top-F children by (s desc, parent slot asc, child rank asc); slot = position in F_d
  kept = union of F_1..F_D;  tree = top-N of kept by (s desc, depth asc, slot asc)
  parents are re-indexed into tree order (-1 = root), so parent[j] < j.

Readings: "per-depth top-k pruning" is a frontier of F nodes chosen over all
children of the current frontier by path score; the depth-1 parent is the
anchor; log pi is normalised over the full vocabulary of z(parent); the global
top-N ranges over every kept frontier node of every depth, root excluded. Since
log pi <= 0 a child never outranks its parent, so the depth-ascending tie-break
keeps the tree ancestor-closed.

The verify's target forward attends tree-causally: node j sees itself and its
ancestors. ``ancestor_masks`` writes that relation as bit sets, word w of node
j holding bit (a mod 64) for every ancestor-or-self a with a // 64 == w (the
root is implicit and not a bit).

Pinned by: k = 1, F = 1 reduces to the greedy Markov chain; with no pruning on
a tiny vocabulary the tree equals brute-force top-N over all paths by summed
fp64 log-probability; invariants parent[j] < j, ancestor closure, scores
non-increasing along paths, distinct sibling tokens, |F_d| <= F
(tests/test_oracle_pctree.py).
"""
import numpy as np

from .markov import markov_logits, logsumexp_rows


def _topk_tokens(z_row, k):
    """Top-k token ids of one row by (fp32 value desc, id asc); also the fp64 boundary gap."""
    z32 = np.asarray(z_row, dtype=np.float64).astype(np.float32)
    V = z32.shape[0]
    k = min(k, V)
    kth = -np.partition(-z32, k - 1)[k - 1]
    cand = np.flatnonzero(z32 >= kth)
    order = cand[np.lexsort((cand, -z32[cand]))]
    top = order[:k]
    # gap (fp64) between the k-th chosen and the best unchosen token
    if V > k:
        rest = np.ones(V, dtype=bool)
        rest[top] = False
        gap = float(np.asarray(z_row, dtype=np.float64)[top[-1]] -
                    np.max(np.asarray(z_row, dtype=np.float64)[rest]))
    else:
        gap = np.inf
    return top, gap


def expand_request(L_i, U, W, anchor, topk, frontier, topN):
    """PCTree for one request. L_i: [D, V]. Returns (nodes list in tree order, min relative gap)."""
    D, V = L_i.shape
    fr = [dict(tok=int(anchor), score=0.0, id=-1)]
    kept = []
    min_gap = np.inf
    for d in range(1, D + 1):
        toks = np.array([f["tok"] for f in fr], dtype=np.int64)
        z = markov_logits(np.broadcast_to(L_i[d - 1], (len(fr), V)), U, W, toks)
        lse = logsumexp_rows(z)
        cands = []
        for p, f in enumerate(fr):
            top, gap = _topk_tokens(z[p], topk)
            min_gap = min(min_gap, gap / max(1.0, abs(float(z[p, top[-1]]))))
            for r, v in enumerate(top):
                s = f["score"] + (float(z[p, v]) - float(lse[p]))
                cands.append((s, p, r, int(v)))
        cands.sort(key=lambda c: (-c[0], c[1], c[2]))
        for a, b in zip(cands[:frontier], cands[1:frontier + 1]):
            min_gap = min(min_gap, (a[0] - b[0]) / max(1.0, abs(a[0])))
        new_fr = []
        for slot, (s, p, r, v) in enumerate(cands[:frontier]):
            node = dict(id=len(kept), tok=v, parent=fr[p]["id"], depth=d, score=s, slot=slot)
            kept.append(node)
            new_fr.append(dict(tok=v, score=s, id=node["id"]))
        fr = new_fr
    ordered = sorted(kept, key=lambda n: (-n["score"], n["depth"], n["slot"]))
    for a, b in zip(ordered[:topN], ordered[1:topN + 1]):
        min_gap = min(min_gap, (a["score"] - b["score"]) / max(1.0, abs(a["score"])))
    tree = ordered[:topN]
    pos = {n["id"]: j for j, n in enumerate(tree)}
    out = []
    for n in tree:
        par = -1 if n["parent"] < 0 else pos[n["parent"]]  # KeyError = not ancestor-closed
        out.append(dict(token=n["tok"], parent=par, depth=n["depth"], score=n["score"]))
    return out, min_gap


def tree_expand(L, U, W, anchor, topk, frontier, topN, requests=None):
    """PCTree for a batch. L: [R, D, V]. Returns dict of [R, topN] arrays (+ n_nodes, min_gap).

    requests: optional subset of request indices to evaluate (rows of the output
    for other requests are left at their fill values).
    """
    L = np.asarray(L)
    R, D, V = L.shape
    tok = np.full((R, topN), -1, dtype=np.int32)
    par = np.full((R, topN), -1, dtype=np.int32)
    dep = np.zeros((R, topN), dtype=np.int32)
    sc = np.zeros((R, topN), dtype=np.float64)
    nn = np.zeros(R, dtype=np.int32)
    gaps = np.full(R, np.inf)
    todo = range(R) if requests is None else requests
    for i in todo:
        nodes, g = expand_request(L[i], U, W, int(anchor[i]), topk, frontier, topN)
        gaps[i] = g
        nn[i] = len(nodes)
        for j, n in enumerate(nodes):
            tok[i, j], par[i, j], dep[i, j], sc[i, j] = n["token"], n["parent"], n["depth"], n["score"]
    return dict(node_token=tok, node_parent=par, node_depth=dep, node_score=sc, n_nodes=nn,
                min_gap=gaps)


def ancestor_masks(node_parent, n_nodes):
    """[R, N, ceil(N/64)] uint64 ancestor-or-self bit sets of the tree nodes (0 past n_nodes)."""
    par = np.asarray(node_parent, dtype=np.int64)
    R, N = par.shape
    Wd = (N + 63) // 64
    out = np.zeros((R, N, Wd), dtype=np.uint64)
    for i in range(R):
        for j in range(int(n_nodes[i])):
            a = j
            while a >= 0:
                out[i, j, a // 64] |= np.uint64(1) << np.uint64(a % 64)
                a = int(par[i, a])
    return out
