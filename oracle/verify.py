"""Rejection-sampling verify, greedy verify and greedy tree walk -- oracle side (test infrastructure).

Follows the DSpark study notes (pages.layerx.co.jp), section 1 "Background":
drafts are checked left to right, each with an acceptance probability; the
first rejected position and everything after it are dropped; one bonus token
is appended; rejection sampling keeps the target distribution exactly. Section
3 / Figure 1 of the same notes: when draft G is rejected the target writes the
corrected token G*. The SGLang article (winzheng.jp), sections "three verify
modes" and "Ragged verify", fixes the packed layout: request i owns rows
cu_seqlens[i] .. cu_seqlens[i+1]-1 of the target buffer, its anchor first.

Per request i with window n = cu_seqlens[i+1] - cu_seqlens[i] - 1 and
k = 1..n:  p_k = softmax(t_{i,k-1} / T) (target row that predicts position k),
q_k = softmax(d_{i,k} / T) (draft distribution of position k),
accept x_k iff u_k < p_k(x_k) / q_k(x_k) (i.e. with probability min(1, p/q)).
At the first rejection the token is drawn from norm(max(0, p_k - q_k)) with
u'_k; if all n are accepted the bonus is drawn from p_{n+1} with u'_{n+1}.
T = 0 means greedy: x_k is accepted iff it equals argmax t_{i,k-1} and the
token written at the stop is that argmax.

Readings where the pages are silent: the accept formula (stripped from the
extracted text) is min(1, p/q) with a strict "u < ratio"; the residual and
bonus draws are inverse-CDF draws over ascending token id (smallest v whose
cumulative weight exceeds u' times the total; if rounding leaves none, the last
v with positive weight; an all-zero residual falls back to p); the same
temperature divides target and draft logits; uniforms come from Philox4x64-10
keyed by (seed, 0) at counter (round, request id, position, 0), word 0 for u_k
and word 1 for u'_k. All arithmetic is fp64 with two-pass log-sum-exp.

Pinned by: greedy = argmax-prefix matching; q == p accepts the whole block;
closed-form expected accepted length (1 - a^(K+1)) / (1 - a) for i.i.d.
acceptance a; exact enumeration and Monte-Carlo chi-square on a vocabulary of 8
showing the committed token's law equals the target's; position-1 acceptance
rate equal to sum_v min(p_v, q_v); the Figure-1 fixture (tests/test_oracle_verify.py).

The exact token drawn under sampling is fixed by the inverse-CDF convention,
not by the pages: parity unpinned for token identity under sampling (its law is
pinned by the tests above).
"""
import numpy as np

from . import philox


def log_softmax(row, temperature):
    """fp64 log-softmax of row / T, two-pass (max, then sum of exp)."""
    s = np.asarray(row, dtype=np.float64) / float(temperature)
    m = np.max(s)
    return s - (m + np.log(np.sum(np.exp(s - m))))


def argmax_lowest(row):
    """Index of the largest value, lowest index on ties (+0 and -0 compare equal)."""
    row = np.asarray(row)
    return int(np.flatnonzero(row == row.max())[0])


def inverse_cdf(weights, u):
    """Smallest v with sum_{w<=v} weights_w > u * sum(weights); returns (v, relative margin).

    The margin is the distance of u*total from the nearest CDF boundary of the
    chosen v, divided by the total (used to recognise near-ties).
    """
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    total = c[-1]
    target = u * total
    v = int(np.searchsorted(c, target, side="right"))
    if v >= w.shape[0]:
        v = int(np.flatnonzero(w > 0)[-1])
    lo = c[v - 1] if v > 0 else 0.0
    margin = min(target - lo, c[v] - target) / total
    return v, float(margin)


def _sample(p_row, q_row, u):
    """Residual draw norm(max(0, p - q)); p itself when q_row is None (bonus) or residual is empty."""
    if q_row is not None:
        r = np.maximum(0.0, p_row - q_row)
        if np.sum(r) > 0:
            return inverse_cdf(r, u)
    return inverse_cdf(p_row, u)


def verify_chain(tgt, cu_seqlens, drf, draft_tok, temperature, seed=0, rnd=0, req_id=None,
                 forced_len=None, cap=None):
    """Chain verify over a packed target buffer.

    tgt: [T_rows, V] logits (exact float values of the stored dtype);
    drf: [R, K, V]; draft_tok: [R, K]; cu_seqlens: [R+1].
    forced_len: optional [R]; when given, request i follows accept for
    k <= forced_len[i] and reject at forced_len[i] + 1 (replay of another
    implementation's decisions over the whole packed window); ``agree`` then
    tells where that differs from the oracle's own decision.
    cap: optional [R] commit windows (the SGLang article's cap-accept mode):
    the decisions run over the whole packed window n_i, ``ceiling`` reports how
    many drafts that full verify accepts, and only the first c_i = min(cap_i, n_i)
    positions are committed: a rejection at k <= c_i stops there as usual; if the
    first c_i drafts are all accepted, the bonus is drawn from p_{c_i+1} with the
    sampling uniform of position c_i + 1 -- exactly what verifying the window c_i
    alone commits (compact mode), while the full block exposes the ceiling.

    Returns dict(accepted_len [R], out_tokens [R, K+1] (-1 padded), stop_pos [R],
    ceiling [R] (drafts accepted over the whole window), p_x, q_x [R, K] (every
    window position; 0 beyond the window and under greedy), ratio [R, K] (p/q at
    x, 0 where not computed), accept_margin [R, K] (|u - ratio|, +inf where not
    decided), sample_margin [R], resid_mass [R] (sum of max(0, p - q) at the stop
    when the token there is a residual draw, 0 for a bonus draw), agree [R] bool).
    """
    tgt = np.asarray(tgt)
    drf = np.asarray(drf)
    draft_tok = np.asarray(draft_tok, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    R, K = draft_tok.shape
    rid = np.arange(R) if req_id is None else np.asarray(req_id, dtype=np.int64)
    greedy = float(temperature) == 0.0
    u_acc, u_smp = philox.verify_uniforms(seed, rnd, rid, K + 1)
    acc_len = np.zeros(R, dtype=np.int32)
    out = np.full((R, K + 1), -1, dtype=np.int32)
    stop = np.zeros(R, dtype=np.int32)
    ceiling = np.zeros(R, dtype=np.int32)
    p_x = np.zeros((R, K), dtype=np.float64)
    q_x = np.zeros((R, K), dtype=np.float64)
    ratio_out = np.zeros((R, K), dtype=np.float64)
    acc_margin = np.full((R, K), np.inf)
    smp_margin = np.full(R, np.inf)
    resid_mass = np.zeros(R, dtype=np.float64)
    agree = np.ones(R, dtype=bool)
    for i in range(R):
        base = int(cu[i])
        n = int(cu[i + 1]) - base - 1
        assert 0 <= n <= K
        ratio = np.zeros(n + 1)
        if not greedy:
            # p_k(x_k), q_k(x_k) and the ratio for every position of the window
            for k in range(1, n + 1):
                x = int(draft_tok[i, k - 1])
                lp = log_softmax(tgt[base + k - 1], temperature)
                lq = log_softmax(drf[i, k - 1], temperature)
                p_x[i, k - 1] = np.exp(lp[x])
                q_x[i, k - 1] = np.exp(lq[x])
                ratio[k] = np.exp(lp[x] - lq[x])
                ratio_out[i, k - 1] = ratio[k]
        stopped_at = None
        for k in range(1, n + 1):
            x = int(draft_tok[i, k - 1])
            if greedy:
                own = x == argmax_lowest(tgt[base + k - 1])
            else:
                own = bool(u_acc[i, k - 1] < ratio[k])
                acc_margin[i, k - 1] = abs(u_acc[i, k - 1] - ratio[k])
            take = own if forced_len is None else (k <= int(forced_len[i]))
            if take != own:
                agree[i] = False
            if take:
                continue
            stopped_at = k
            break
        if stopped_at is None:
            k = n + 1
            if forced_len is not None and int(forced_len[i]) != n:
                agree[i] = False
        else:
            k = stopped_at
        ceiling[i] = k - 1
        c = n if cap is None else max(0, min(int(cap[i]), n))
        if k > c + 1:  # the first c drafts are all accepted: commit them and draw the bonus after them
            k = c + 1
        for j in range(1, k):
            out[i, j - 1] = int(draft_tok[i, j - 1])
        acc_len[i] = k - 1
        stop[i] = k
        if greedy:
            out[i, k - 1] = argmax_lowest(tgt[base + k - 1])
        else:
            p = np.exp(log_softmax(tgt[base + k - 1], temperature))
            rejected = ceiling[i] + 1 <= c  # a rejection inside the commit window: residual draw
            q = np.exp(log_softmax(drf[i, k - 1], temperature)) if rejected else None
            if rejected:
                resid_mass[i] = float(np.sum(np.maximum(0.0, p - q)))
            v, mg = _sample(p, q, u_smp[i, k - 1])
            out[i, k - 1] = v
            smp_margin[i] = mg
    return dict(accepted_len=acc_len, out_tokens=out, stop_pos=stop, ceiling=ceiling, p_x=p_x, q_x=q_x,
                ratio=ratio_out, accept_margin=acc_margin, sample_margin=smp_margin, resid_mass=resid_mass,
                agree=agree)


def verify_tree_greedy(tgt, cu_seqlens, node_token, node_parent):
    """Greedy walk of a draft tree (PCTree article: one target forward verifies the tree).

    Request i owns packed rows cu[i] (root = anchor) and cu[i] + 1 + j (node j),
    n_nodes = cu[i+1] - cu[i] - 1. From the root, move to the child whose token
    equals argmax of the current node's target row; stop when no child matches;
    the bonus is that argmax.

    Returns dict(accepted_len [R], out_tokens [R, N+1] (-1 padded), stop_node [R]
    (-1 = root)).
    """
    tgt = np.asarray(tgt)
    node_token = np.asarray(node_token, dtype=np.int64)
    node_parent = np.asarray(node_parent, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    R, N = node_token.shape
    acc_len = np.zeros(R, dtype=np.int32)
    out = np.full((R, N + 1), -1, dtype=np.int32)
    stop = np.full(R, -1, dtype=np.int32)
    for i in range(R):
        base = int(cu[i])
        nn = int(cu[i + 1]) - base - 1
        cur = -1
        path = []
        while True:
            a = argmax_lowest(tgt[base + 1 + cur])
            nxt = -1
            for j in range(nn):
                if node_parent[i, j] == cur and node_token[i, j] == a:
                    nxt = j
                    break
            if nxt < 0:
                break
            path.append(nxt)
            cur = nxt
        for d, j in enumerate(path):
            out[i, d] = node_token[i, j]
        out[i, len(path)] = a
        acc_len[i] = len(path)
        stop[i] = cur
    return dict(accepted_len=acc_len, out_tokens=out, stop_node=stop)
