"""RNN sequential head -- oracle side (test infrastructure).

Follows the DSpark study notes (pages.layerx.co.jp), section 4, "RNN head": the
Markov head remembers only the previous token; the RNN head keeps an internal memo
s that accumulates everything drafted so far, and updates it once per position from
the previous memo, the previous token and the current internal state of the
parallel backbone. As for the Markov head, the position's logits are the base
logits plus the head's correction, normalised over the whole vocabulary, and the
token is the most probable one.

Reading (the update's formula is stripped from the extracted text; the plainest
recurrent cell that uses exactly those three inputs, with the correction a rank-r
projection onto the vocabulary like the Markov head's second factor):
    s_0 = 0
    s_d = tanh(s_{d-1} A + E[y_{d-1}] + h_d G + b)        (memo, r entries, fp64)
    z_d = L_d + bf16(s_d) W_o                              (correction: rank r)
    y_d = argmax z_d (lowest id on exact ties),  log q_d = z_{y_d} - logsumexp(z_d)
with y_0 the anchor, h_d the backbone's internal state of position d (H entries),
A [r, r], E [V, r], G [H, r], b [r], W_o [r, V]. The memo enters the vocabulary
projection rounded to bfloat16 (nearest, ties to even), the precision of the
projection's weights; it is carried in fp64 from step to step.

Pinned by: with A = 0 and G = 0 (no recurrence, no state) the head is a Markov head
whose first factor is the rounded tanh(E + b) (oracle.markov.chain on that factor);
W_o = 0 gives argmax L; a two-step fixture in which the third position's choice
depends on the first drafted token, which a Markov head cannot see
(tests/golden/rnn_memory.json); the memo equals an independent step-by-step
evaluation of the recurrence on a tiny case (tests/test_oracle_rnn.py).
"""
import numpy as np

from .markov import logsumexp_rows, round_bf16, top2_margin

# a memo entry this close to a bf16 rounding midpoint (relative to max(1, |s|)) may round
# the other way in another implementation's fp64 arithmetic: a rounding near-tie
MEMO_BAND = 1e-12


def rnn_chain(L, h, A, E, G, b, Wo, anchor, n_steps=None, forced=None, memo_choice=None):
    """Greedy chain with the RNN head. L [R, B, V], h [R, B, H]; returns dict(y [R, n],
    logq [R, n], logq_forced [R, n], memo [R, n, r] fp64, memo_bf16 [R, n, r] fp64 values,
    memo_tie [R, n, r] bool, margin [R, n] (fp64 top-2 gap), zmax [R, n]).

    forced: optional [R, n] tokens each step conditions on (replay of another
    implementation's choices). memo_choice: optional [R, n, r] bf16 values another
    implementation used for the projection; at rounding near-ties of the memo the oracle
    takes that value (when it is one of the two candidates), elsewhere its own.
    """
    L = np.asarray(L)
    R, B, V = L.shape
    n = B if n_steps is None else int(n_steps)
    A = np.asarray(A, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    b = np.zeros(A.shape[0]) if b is None else np.asarray(b, dtype=np.float64)
    Wo = np.asarray(Wo, dtype=np.float64)
    h = np.asarray(h)
    r = A.shape[0]
    y = np.zeros((R, n), dtype=np.int64)
    logq = np.zeros((R, n))
    logq_forced = np.zeros((R, n))
    memo = np.zeros((R, n, r))
    memo_bf = np.zeros((R, n, r))
    memo_tie = np.zeros((R, n, r), dtype=bool)
    margin = np.zeros((R, n))
    zmax = np.zeros((R, n))
    s = np.zeros((R, r))
    prev = np.asarray(anchor, dtype=np.int64).copy()
    for d in range(n):
        s = np.tanh(s @ A + E[prev] + np.asarray(h[:, d], dtype=np.float64) @ G + b)
        sb, gap, ulp = round_bf16(s)
        tie = gap < MEMO_BAND * np.maximum(1.0, np.abs(s))
        if memo_choice is not None and tie.any():
            other = np.asarray(memo_choice, dtype=np.float64)[:, d]
            lo = np.where(sb > s, sb - ulp, sb)
            hi = np.where(sb > s, sb, sb + ulp)
            ok = tie & ((other == lo) | (other == hi))
            sb = np.where(ok, other, sb)
        memo[:, d], memo_bf[:, d], memo_tie[:, d] = s, sb, tie
        z = np.asarray(L[:, d], dtype=np.float64) + sb @ Wo
        yd = np.argmax(z, axis=-1)
        lse = logsumexp_rows(z)
        y[:, d] = yd
        logq[:, d] = z[np.arange(R), yd] - lse
        margin[:, d], zmax[:, d] = top2_margin(z)
        prev = yd if forced is None else np.asarray(forced, dtype=np.int64)[:, d]
        logq_forced[:, d] = z[np.arange(R), prev] - lse
    return dict(y=y, logq=logq, logq_forced=logq_forced, memo=memo, memo_bf16=memo_bf, memo_tie=memo_tie,
                margin=margin, zmax=zmax)
