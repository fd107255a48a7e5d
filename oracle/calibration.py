"""Calibration of the confidences against verify outcomes -- oracle side (test infrastructure).

The SGLang article (winzheng.jp, DSpark in SGLang), section on observability:
beside the acceptance ceiling that cap-accept exposes, the serving system reports
per-request confidences and calibration metrics such as ECE. The DSpark study
notes (section 5.1) define what a confidence predicts: c_{i,k} is the probability
that draft position k survives verification given that every earlier position of
the request was accepted.

So the outcome of position k of request i is observed only where the verify
decided it: with window n_i and m_i drafts accepted over the decided window
(the accepted length, or under cap-accept the full-window ceiling), positions
k = 1..m_i are accepted (outcome 1) and, if m_i < n_i, position m_i + 1 is the
first rejection (outcome 0); later positions were never decided and carry no
outcome. A request whose verify faulted (accepted length -1) has none.

Expected calibration error over a set of (confidence, outcome) pairs with B
equal-width bins of [0, 1] (bin b = [b/B, (b+1)/B), the last one closed; bin
index floor(c * B) computed in fp64, exact for fp32 confidences):
    ECE = sum_b (n_b / n) * |mean outcome in b - mean confidence in b|,
0 for an empty set. Reported per request (over its observed positions) and for
the batch (over all observed positions), in fp64.

Readings: the pages name ECE without a formula or bin count; the standard
equal-width binned form above is taken, B a parameter (10 by default).

Pinned by hand-computed cases: perfect calibration gives 0, a single rejected
position at confidence c gives c, a worked two-bin batch (tests/golden/ece_case.json),
and invariance of the per-request value under the order of positions
(tests/test_oracle_calibration.py).
"""
import numpy as np


def observations(conf_row, window, decided):
    """(confidences, outcomes) of the positions the verify decided for one request."""
    n, m = int(window), int(decided)
    if m < 0 or n <= 0:
        return np.zeros(0), np.zeros(0)
    last = min(n, m + 1)
    c = np.asarray(conf_row, dtype=np.float64)[:last]
    o = np.array([1.0 if k < m else 0.0 for k in range(last)])
    return c, o


def bin_index(c, n_bins):
    return np.minimum(n_bins - 1, np.floor(np.asarray(c, dtype=np.float64) * n_bins).astype(np.int64))


def ece(c, o, n_bins=10):
    """Binned expected calibration error of confidences c against outcomes o."""
    c = np.asarray(c, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    n = c.shape[0]
    if n == 0:
        return 0.0
    b = bin_index(c, n_bins)
    total = 0.0
    for j in range(n_bins):
        sel = b == j
        nb = int(sel.sum())
        if nb:
            total += (nb / n) * abs(o[sel].mean() - c[sel].mean())
    return float(total)


def verify_ece(conf, cu_seqlens, decided, n_bins=10):
    """Per-request and batch ECE of conf [R, K] against a verify's decisions.

    cu_seqlens [R+1] gives each window n_i = cu[i+1] - cu[i] - 1; decided [R] is the
    accepted length (or the cap-accept ceiling). Returns dict(ece [R], n_obs [R],
    ece_batch, bin_count [B], bin_conf [B], bin_out [B] (batch sums per bin)).
    """
    conf = np.asarray(conf)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    R = conf.shape[0]
    e = np.zeros(R)
    nobs = np.zeros(R, dtype=np.int64)
    allc, allo = [], []
    for i in range(R):
        c, o = observations(conf[i], cu[i + 1] - cu[i] - 1, decided[i])
        e[i] = ece(c, o, n_bins)
        nobs[i] = c.shape[0]
        allc.append(c)
        allo.append(o)
    c = np.concatenate(allc) if allc else np.zeros(0)
    o = np.concatenate(allo) if allo else np.zeros(0)
    b = bin_index(c, n_bins)
    cnt = np.array([(b == j).sum() for j in range(n_bins)], dtype=np.float64)
    sc = np.array([c[b == j].sum() for j in range(n_bins)])
    so = np.array([o[b == j].sum() for j in range(n_bins)])
    return dict(ece=e, n_obs=nobs, ece_batch=ece(c, o, n_bins), bin_count=cnt, bin_conf=sc, bin_out=so)
