"""Markov-head sequential stage, greedy chain -- oracle side (test infrastructure).

Follows the DSpark study notes (pages.layerx.co.jp), section 4
"Semi-Autoregressive Generation": the parallel backbone emits base logits L_d
for every block position in one pass; then, left to right, the sequential head
adds a correction that depends on the token already chosen at the previous
position, and the position's distribution is the softmax of (base logits +
correction) over the whole vocabulary. The Markov head makes the correction a
function of the previous token only, approximating the V x V transition table
by the product of two small factors. The PCTree article (qiita.com) writes the
same step as z_d = L_d + Markov(y_{d-1}) with the most probable token chosen.

So, with y_0 = the anchor token and factors U [V, r], W [r, V]:
    z_d = L_d + U[y_{d-1}] @ W,   y_d = argmax_v z_d[v],   d = 1..B,
and log q_d(y_d) = z_d[y_d] - logsumexp(z_d).

Readings: the selection rule (stripped from the extracted text) is argmax, as
the PCTree article states; the rank is a parameter (256 in the workloads). z is
computed in fp64 and the argmax is taken on those fp64 values, lowest token id
on exact ties. An implementation that decides in lower precision may differ
only where the winner and the runner-up are closer than its rounding error;
``top2_margin`` reports that gap so a checker can recognise such near-ties.

Sampled chain (the draft side of the full draft -> schedule -> pack -> verify
cycle; SGLang article, "Ragged verify", and the notes' section 1: the verifier
needs the draft distribution q of every drafted position): the step's logits are
emitted as bf16, ẑ_d = bf16(z_d) (round to nearest, ties to even, from the exact
value), q_d = softmax(ẑ_d / T), and y_d is the inverse-CDF draw from q_d over
ascending token ids with the Philox uniform of (round, request id, d, stream 1).
Drawing from the emitted bf16 rows makes the verify step's q exactly the law the
token came from, which rejection sampling needs.

Pinned by: W = 0 reduces each step to numpy's argmax of L_d; the rank-r term
equals an independent fp64 dot-product evaluation; the "of course / no problem"
fixture of the notes' section 2 and Figure 2 (a tie in L_2 resolved toward the
token the previous choice boosts); logq normalisation; for the sampled chain,
bf16 rounding equal to the integer rounding of float32 inputs and to the nearer
of the two enumerated bf16 neighbours of fp64 inputs, the two-token logistic
law of the draw, and the T -> 0 limit equal to the argmax of the rounded row
(tests/test_oracle_markov.py).
"""
import numpy as np

from . import philox
from .verify import inverse_cdf


def markov_logits(L_row, U, W, prev_tok):
    """z = L_d + U[prev] @ W in fp64, for a batch of rows: L_row [n, V], prev_tok [n]."""
    U64 = np.asarray(U, dtype=np.float64)
    W64 = np.asarray(W, dtype=np.float64)
    prev = np.asarray(prev_tok, dtype=np.int64)
    return np.asarray(L_row, dtype=np.float64) + U64[prev] @ W64


def logsumexp_rows(z):
    m = np.max(z, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))[..., 0]


def decide_argmax(z):
    """argmax of each fp64 row of z, lowest index on ties."""
    return np.argmax(np.asarray(z, dtype=np.float64), axis=-1)  # numpy returns the first maximal index


def top2_margin(z):
    """fp64 gap between the best and second-best entry of each row (near-tie test)."""
    part = -np.partition(-np.asarray(z, dtype=np.float64), 1, axis=-1)
    return part[..., 0] - part[..., 1], part[..., 0]


def chain(L, U, W, anchor, n_steps=None, forced=None, want_margin=False):
    """Greedy Markov chain: L [R, B, V]; returns dict(y [R, n], logq [R, n]).

    forced: optional [R, n] tokens; when given, step d conditions on forced[:, d-1]
    instead of the oracle's own choice (replay of another implementation), so
    every step can be checked locally.
    """
    L = np.asarray(L)
    R, B, V = L.shape
    n = B if n_steps is None else int(n_steps)
    y = np.zeros((R, n), dtype=np.int64)
    logq = np.zeros((R, n), dtype=np.float64)
    logq_forced = np.zeros((R, n), dtype=np.float64)
    margin = np.zeros((R, n), dtype=np.float64)
    zmax = np.zeros((R, n), dtype=np.float64)
    prev = np.asarray(anchor, dtype=np.int64).copy()
    for d in range(n):
        z = markov_logits(L[:, d, :], U, W, prev)
        yd = decide_argmax(z)
        y[:, d] = yd
        logq[:, d] = z[np.arange(R), yd] - logsumexp_rows(z)
        if want_margin:
            margin[:, d], zmax[:, d] = top2_margin(z)
        prev = yd if forced is None else np.asarray(forced, dtype=np.int64)[:, d]
        logq_forced[:, d] = z[np.arange(R), prev] - logsumexp_rows(z)
    res = dict(y=y, logq=logq)
    if forced is not None:
        res.update(logq_forced=logq_forced)
    if want_margin:
        res.update(margin=margin, zmax=zmax)
    return res


def round_bf16(z):
    """Round fp64 values to the nearest bfloat16 value (ties to even).

    Returns (values as fp64, distance of each input to the nearest rounding
    midpoint, one bf16 unit in the last place at each input). bfloat16 keeps 8
    significant bits: with z = m * 2^e, 0.5 <= |m| < 1, the kept significand is
    m * 2^8 rounded to an integer. A masked logit (-inf) rounds to itself, with
    no midpoint near it (gap +inf) and unit 0.
    """
    z = np.asarray(z, dtype=np.float64)
    masked = np.isneginf(z)
    assert np.all(np.isfinite(z) | masked)
    zf = np.where(masked, 0.0, z)
    m, e = np.frexp(zf)
    s = m * 256.0
    r = np.rint(s)  # nearest integer, ties to even
    out = np.where(masked, -np.inf, np.ldexp(r / 256.0, e))
    a = np.abs(s)
    mid_gap = np.where(masked, np.inf, np.ldexp(np.abs((a - np.floor(a)) - 0.5) / 256.0, e))
    ulp = np.where(masked, 0.0, np.ldexp(np.full_like(zf, 1.0 / 256.0), e))
    return out, mid_gap, ulp


# a bf16 rounding whose input lies this close to a midpoint (relative to max(1, |z|)) may
# round the other way in fp32 arithmetic: counted as a near-tie of the emitted row
ROUND_BAND = 1e-5


def chain_sampled(L, U, W, anchor, temperature, seed=0, rnd=0, req_id=None, n_steps=None, forced=None):
    """Sampled Markov chain: L [R, B, V]; step d draws y_d from softmax(bf16(z_d) / T).

    forced: optional [R, n] tokens to condition on (replay of another
    implementation's draws), as in ``chain``.
    Returns dict(y [R, n], logq [R, n] (of the oracle's own draw), logq_forced,
    zhat [R, n, V] fp64 values of the emitted bf16 rows, round_tie [R, n, V] bool
    (inputs within ROUND_BAND of a rounding midpoint), sample_margin [R, n]
    (distance of u * total to the nearest CDF boundary over the total), and the
    bounds a checker needs when another implementation's emitted row differs at
    those near-midpoint entries, each by at most dev_v = one unit + ROUND_BAND *
    max(1, |z_v|):
      eps [R, n]       = sum over tie entries of q_v * expm1(dev_v / T). Every weight
                         w_v = exp(zhat_v / T) moves by a factor within exp(+-dev_v / T),
                         so the total S moves by at most eps * S.
      tie_shift [R, n] = 2 eps / (1 - eps): bound on the move of the normalised CDF at any
                         point (|C'/S' - C/S| <= (|C' - C| + C |S' - S| / S) / S'), i.e. of
                         the draw's margin; also bounds the L1 distance sum |q'_v - q_v|.
      tok_dev [R, n]   = dev of the token the next step conditions on (its own draw, or
                         the forced one), 0 if that entry is not a near-midpoint one: its
                         probability moves by a factor within exp(+-(tok_dev / T + log(1/(1-eps)))).
    """
    L = np.asarray(L)
    R, B, V = L.shape
    n = B if n_steps is None else int(n_steps)
    T = float(temperature)
    assert T > 0
    rid = np.arange(R) if req_id is None else np.asarray(req_id, dtype=np.int64)
    y = np.zeros((R, n), dtype=np.int64)
    logq = np.zeros((R, n))
    logq_forced = np.zeros((R, n))
    zhat = np.zeros((R, n, V))
    round_tie = np.zeros((R, n, V), dtype=bool)
    margin = np.zeros((R, n))
    shift = np.zeros((R, n))
    eps = np.zeros((R, n))
    tok_dev = np.zeros((R, n))
    prev = np.asarray(anchor, dtype=np.int64).copy()
    for d in range(n):
        z = markov_logits(L[:, d, :], U, W, prev)
        zh, gap, ulp = round_bf16(z)
        devs = []
        zhat[:, d] = zh
        tie = gap < ROUND_BAND * np.maximum(1.0, np.abs(z))
        round_tie[:, d] = tie
        u = philox.draft_uniforms(seed, rnd, rid, d + 1)
        for i in range(R):
            s = zh[i] / T
            mx = np.max(s)
            w = np.exp(s - mx)
            lse = mx + np.log(np.sum(w))
            v, mg = inverse_cdf(w, u[i])
            y[i, d] = v
            margin[i, d] = mg
            logq[i, d] = s[v] - lse
            q = w / np.sum(w)
            # a near-midpoint entry computed in fp32 may land up to one unit plus the band away
            dev_row = np.where(tie[i], ulp[i] + ROUND_BAND * np.maximum(1.0, np.abs(z[i])), 0.0)
            e = float(np.sum(q * np.expm1(dev_row / T)))
            eps[i, d] = e
            shift[i, d] = 2.0 * e / (1.0 - e) if e < 1.0 else np.inf
            devs.append(dev_row)
        prev = y[:, d] if forced is None else np.asarray(forced, dtype=np.int64)[:, d]
        for i in range(R):
            tok_dev[i, d] = devs[i][prev[i]]
        logq_forced[:, d] = zh[np.arange(R), prev] / T - (
            np.max(zh / T, axis=-1) + np.log(np.sum(np.exp(zh / T - np.max(zh / T, axis=-1, keepdims=True)),
                                                   axis=-1)))
    return dict(y=y, logq=logq, logq_forced=logq_forced, zhat=zhat, round_tie=round_tie,
                sample_margin=margin, tie_shift=shift, eps=eps, tok_dev=tok_dev)
