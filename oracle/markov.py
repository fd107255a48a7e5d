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
computed in fp64; the argmax decision is taken on z rounded to fp32, the
precision the GPU path decides in, lowest token id on ties.

Pinned by: W = 0 reduces each step to numpy's argmax of L_d; the rank-r term
equals an independent fp64 dot-product evaluation; the "of course / no problem"
fixture of the notes' section 2 and Figure 2 (a tie in L_2 resolved toward the
token the previous choice boosts); logq normalisation (tests/test_oracle_markov.py).
"""
import numpy as np


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
    """argmax of each row of z rounded to fp32, lowest index on ties."""
    z32 = np.asarray(z, dtype=np.float64).astype(np.float32)
    return np.argmax(z32, axis=-1)  # numpy returns the first maximal index


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
