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
      children = top-k tokens of z by (fp64 z desc, token asc)
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

Replay of another implementation (the parity checker's hook): given that
implementation's tree as a set of token paths, every cut the expansion makes --
a parent's top-k, a depth's frontier, the global top-N and the order of the
output -- is taken as above except inside a near-tie run, a stretch of the
sorted candidates whose neighbouring values differ by less than
band * max(1, |value|). Inside such a run the candidates the other tree holds
go first (in that tree's order), so a decision that rounding could have taken
either way follows the other implementation, and everything downstream of it
is still computed here. Each cut this changes is counted as a near-tie.

Pinned by: k = 1, F = 1 reduces to the greedy Markov chain; with no pruning on
a tiny vocabulary the tree equals brute-force top-N over all paths by summed
fp64 log-probability; invariants parent[j] < j, ancestor closure, scores
non-increasing along paths, distinct sibling tokens, |F_d| <= F; the replay
leaves a tree unchanged when the preferred tree is the oracle's own, and takes
the other branch exactly at a planted near-tie (tests/test_oracle_pctree.py).
"""
import numpy as np

from .markov import markov_logits, logsumexp_rows


def _near(a, b, band):
    """Neighbouring sorted values a >= b form a near-tie."""
    return (a - b) < band * max(1.0, abs(a))


def _run_around(vals, cut, band):
    """(start, end) of the near-tie run holding sorted positions cut-1 and cut (descending
    values), or None when the values at the cut are not near-tied. end is exclusive; a run
    reaching the end of vals returns end = len(vals)."""
    n = len(vals)
    if cut <= 0 or cut >= n or not _near(vals[cut - 1], vals[cut], band):
        return None
    a = cut - 1
    while a > 0 and _near(vals[a - 1], vals[a], band):
        a -= 1
    b = cut + 1
    while b < n and _near(vals[b - 1], vals[b], band):
        b += 1
    return a, b


def _cut(items, vals, keep, band, pref):
    """First `keep` of items (sorted by the strict key, vals descending alongside). Inside the
    near-tie run straddling the cut, items with a smaller pref(item) are kept first; the kept
    items stay in the strict order. Returns (kept items, changed)."""
    keep = min(keep, len(items))
    run = None if pref is None else _run_around(vals, keep, band)
    if run is None:
        return list(items[:keep]), False
    a, b = run
    inside = sorted(range(a, b), key=lambda j: (pref(items[j]), j))
    chosen = set(range(a)) | set(inside[:keep - a])
    kept = [items[j] for j in sorted(chosen)]
    return kept, sorted(chosen) != list(range(keep))


def _topk_tokens(z_row, k, band=0.0, pref=None):
    """Top-k token ids of one fp64 row by (value desc, id asc); also the relative gap at the
    cut (k-th chosen vs best unchosen) and whether a near-tie replay changed the choice."""
    z = np.asarray(z_row, dtype=np.float64)
    V = z.shape[0]
    k = min(k, V)
    m = min(V, k + 8)
    while True:
        idx = np.argpartition(-z, m - 1)[:m] if m < V else np.arange(V)
        order = idx[np.lexsort((idx, -z[idx]))]
        vals = z[order]
        run = _run_around(vals, k, band) if (pref is not None and m > k) else None
        # an exact tie or a run reaching the end of the partial list needs more candidates
        if m < V and (vals[m - 1] == vals[k - 1] or (run is not None and run[1] == m)):
            m = min(V, 2 * m)
            continue
        break
    gap = (vals[k - 1] - vals[k]) / max(1.0, abs(vals[k - 1])) if m > k else np.inf
    top, changed = _cut(list(order), vals, k, band, pref)
    return np.asarray(top, dtype=np.int64), gap, changed


def _path_prefs(prefer):
    """Preference rank of a node path (tuple of tokens from depth 1) from another tree given
    as (node_token, node_parent, n_nodes) of one request: its index there, +inf if absent."""
    if prefer is None:
        return None
    tok, par, n = prefer
    paths = {}
    for j in range(int(n)):
        pth, a = [], j
        while a >= 0:
            pth.append(int(tok[a]))
            a = int(par[a])
        paths[tuple(reversed(pth))] = j
    return lambda path: paths.get(path, np.inf)


def expand_request(L_i, U, W, anchor, topk, frontier, topN, prefer=None, band=1e-6):
    """PCTree for one request. L_i: [D, V].

    prefer: optional (node_token [N], node_parent [N], n_nodes) of another
    implementation's tree for this request, to replay its near-tie decisions.
    Returns (nodes in tree order, min relative gap over the cuts, near-ties taken
    from `prefer`, decisions made).
    """
    D, V = L_i.shape
    rank = _path_prefs(prefer)
    fr = [dict(tok=int(anchor), score=0.0, id=-1, path=())]
    kept = []
    min_gap = np.inf
    replays = 0
    decisions = 0
    for d in range(1, D + 1):
        toks = np.array([f["tok"] for f in fr], dtype=np.int64)
        z = markov_logits(np.broadcast_to(L_i[d - 1], (len(fr), V)), U, W, toks)
        lse = logsumexp_rows(z)
        cands = []
        for p, f in enumerate(fr):
            pref_tok = None if rank is None else (lambda v, fp=f["path"]: rank(fp + (int(v),)))
            top, gap, changed = _topk_tokens(z[p], topk, band, pref_tok)
            min_gap = min(min_gap, gap)
            replays += int(changed)
            decisions += 1
            for r, v in enumerate(top):
                s = f["score"] + (float(z[p, v]) - float(lse[p]))
                cands.append((s, p, r, int(v), f["path"] + (int(v),)))
        cands.sort(key=lambda c: (-c[0], c[1], c[2]))
        svals = [c[0] for c in cands]
        for a, b in zip(svals[:frontier], svals[1:frontier + 1]):
            min_gap = min(min_gap, (a - b) / max(1.0, abs(a)))
        chosen, changed = _cut(cands, svals, frontier, band, None if rank is None else (lambda c: rank(c[4])))
        replays += int(changed)
        decisions += 1
        new_fr = []
        for slot, (s, p, r, v, path) in enumerate(chosen):
            node = dict(id=len(kept), tok=v, parent=fr[p]["id"], depth=d, score=s, slot=slot, path=path)
            kept.append(node)
            new_fr.append(dict(tok=v, score=s, id=node["id"], path=path))
        fr = new_fr
    ordered = sorted(kept, key=lambda n: (-n["score"], n["depth"], n["slot"]))
    for a, b in zip(ordered[:topN], ordered[1:topN + 1]):
        min_gap = min(min_gap, (a["score"] - b["score"]) / max(1.0, abs(a["score"])))
    decisions += 1
    if rank is not None:
        # every near-tie run that reaches into the first topN places follows the other tree
        sv = [n["score"] for n in ordered]
        out_order, j = [], 0
        while j < len(ordered) and j < topN:
            b = j + 1
            while b < len(ordered) and _near(sv[b - 1], sv[b], band):
                b += 1
            run = list(range(j, b))
            re = sorted(run, key=lambda x: (rank(ordered[x]["path"]), x))
            if re[:topN - j] != run[:topN - j]:
                replays += 1
            out_order.extend(re)
            j = b
        ordered = [ordered[x] for x in out_order]
    tree = ordered[:topN]
    pos = {n["id"]: j for j, n in enumerate(tree)}
    out = []
    for j, n in enumerate(tree):
        par = -1 if n["parent"] < 0 else pos[n["parent"]]  # KeyError = not ancestor-closed
        assert par < j
        out.append(dict(token=n["tok"], parent=par, depth=n["depth"], score=n["score"]))
    return out, min_gap, replays, decisions


def tree_expand(L, U, W, anchor, topk, frontier, topN, requests=None, prefer=None, band=1e-6):
    """PCTree for a batch. L: [R, D, V]. Returns dict of [R, topN] arrays (+ n_nodes, min_gap,
    replays and decisions per request).

    requests: optional subset of request indices to evaluate (rows of the output
    for other requests are left at their fill values).
    prefer: optional (node_token [R, N], node_parent [R, N], n_nodes [R]) of another
    implementation's trees, to replay its near-tie decisions (``expand_request``).
    """
    L = np.asarray(L)
    R, D, V = L.shape
    U = np.asarray(U, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    tok = np.full((R, topN), -1, dtype=np.int32)
    par = np.full((R, topN), -1, dtype=np.int32)
    dep = np.zeros((R, topN), dtype=np.int32)
    sc = np.zeros((R, topN), dtype=np.float64)
    nn = np.zeros(R, dtype=np.int32)
    gaps = np.full(R, np.inf)
    reps = np.zeros(R, dtype=np.int64)
    decs = np.zeros(R, dtype=np.int64)
    todo = range(R) if requests is None else requests
    for i in todo:
        pf = None if prefer is None else (prefer[0][i], prefer[1][i], prefer[2][i])
        nodes, g, rp, dc = expand_request(L[i], U, W, int(anchor[i]), topk, frontier, topN, pf, band)
        gaps[i], reps[i], decs[i] = g, rp, dc
        nn[i] = len(nodes)
        for j, n in enumerate(nodes):
            tok[i, j], par[i, j], dep[i, j], sc[i, j] = n["token"], n["parent"], n["depth"], n["score"]
    return dict(node_token=tok, node_parent=par, node_depth=dep, node_score=sc, n_nodes=nn,
                min_gap=gaps, replays=reps, decisions=decs)


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
