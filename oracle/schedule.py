"""Block survival and the hardware-aware prefix scheduler -- oracle side (test infrastructure).

Follows the DSpark study notes (pages.layerx.co.jp), section 5.1 "Confidence
Head" and section 5.2 "Hardware-aware prefix scheduler", and the SGLang article
(winzheng.jp), section "SPS cost table":

* the confidence c_{i,k} is the probability that draft token k of request i
  survives verification given that every earlier token survived (5.1);
* the probability that the prefix up to k survives is the running product
  S_{i,k} = prod_{j<=k} c_{i,j}, non-increasing in k (5.1, 5.2);
* one verify batch of N = sum_i n_i draft tokens is expected to accept
  E = sum_i sum_{k<=n_i} S_{i,k} tokens; throughput is E times steps-per-second
  at N, i.e. E / c(N) for a step-time table c (5.2; the SGLang article fits an
  additive table to raw step time);
* because S is non-increasing in k, the marginal gain of extending request i to
  k is exactly S_{i,k}; sorting every S_{i,k} in descending order and taking
  candidates greedily is optimal and respects the prefix structure (5.2);
* the greedy pass stops the first time throughput would drop, so each decision
  depends only on the prefix already taken (the non-anticipating early stop of
  5.2). The SGLang article's "SPS-argmax" budget and the global search of the
  notes' section 9.2 are the alternative ``MODE_ARGMAX``.

Readings where the pages are silent (formulas are missing from the extracted
text): N counts draft tokens only (anchor rows are a constant absorbed into the
table's intercept); E excludes bonus tokens; a candidate is taken only if
throughput strictly rises; survival is a left-to-right fp64 product; sums are
taken on S quantised to 2^-Q fixed point (Q = min(40, 53 - ceil(log2(R*K))))
so that every partial sum is an exact integer and any summation order gives
the same bits. Ties in the sort are broken by request id, then position.

Pinned by: brute-force maximisation over every window vector for tiny R, K;
closed-form special cases (c = 1, c = 0, flat cost table); the Figure-1 fixture
of the notes (EFGH with an unconfident H); non-anticipation and prefix closure
(tests/test_oracle_schedule.py).
"""
import math

import numpy as np

MODE_EARLY_STOP = 0
MODE_ARGMAX = 1
MODE_TOP_M = 2
MODE_THRESHOLD = 3


def quant_bits(R, K):
    """Fixed-point fraction bits so that R*K quantised survivals sum exactly in fp64."""
    n = max(int(R) * int(K), 1)
    return min(40, 53 - int(math.ceil(math.log2(n))) if n > 1 else 40)


def survival(conf):
    """S_{i,k} = prod_{j<=k} c_{i,j}, multiplied left to right in fp64 (notes 5.1)."""
    conf = np.asarray(conf, dtype=np.float32)
    R, K = conf.shape
    S = np.empty((R, K), dtype=np.float64)
    for i in range(R):
        s = 1.0
        for k in range(K):
            s = s * float(conf[i, k])
            S[i, k] = s
    return S


def quantise(S, Q):
    """floor(S * 2^Q) as Python-exact unsigned integers (S in [0, 1])."""
    return np.floor(S * (2.0 ** Q)).astype(np.uint64)


def additive_cost(a, b, n_max):
    """Additive step-time table c(n) = a + b*n for n = 0..n_max, in fp64 (SGLang article)."""
    n = np.arange(n_max + 1, dtype=np.float64)
    return a + b * n


def sorted_candidates(Sq):
    """Candidate order: S^q descending, then request id ascending, then position ascending."""
    R, K = Sq.shape
    ii, kk = np.meshgrid(np.arange(R), np.arange(K), indexing="ij")
    ii, kk, sq = ii.ravel(), kk.ravel(), Sq.ravel()
    order = sorted(range(R * K), key=lambda j: (-int(sq[j]), int(ii[j]), int(kk[j])))
    return ii[order], kk[order], sq[order]


def schedule_windows(conf, cost, mode=MODE_EARLY_STOP, max_tokens=-1, threshold=0.0):
    """Per-request verify windows n_i chosen by the prefix scheduler (notes 5.2).

    conf: [R, K] float32 confidences; cost: fp64 table, cost[n] = step time when
    n draft tokens are verified (len >= R*K + 1).
    Modes besides the early stop and the global argmax (notes 9.2):
      MODE_TOP_M -- a capacity fixed in advance (notes 9.2: the verify capacity comes
        from confidences two steps old, the ranking from the current survivals): the
        first min(max_tokens, R*K) candidates of the current order (max_tokens < 0:
        all of them);
      MODE_THRESHOLD -- the conventional fixed threshold (notes 5.2 and 8.3,
        threshold 0 = verify the full block): n_i = #{k : S_{i,k} >= threshold},
        compared on the fp64 survival.
    Returns dict(windows [R] int32, survival [R, K] fp64, N, E, J, Q).
    """
    conf = np.asarray(conf, dtype=np.float32)
    cost = np.asarray(cost, dtype=np.float64)
    R, K = conf.shape
    Q = quant_bits(R, K)
    S = survival(conf)
    Sq = quantise(S, Q)
    ci, ck, csq = sorted_candidates(Sq)
    M = R * K if max_tokens is None or max_tokens < 0 else min(R * K, int(max_tokens))
    # exact prefix sums of the quantised survivals
    E = [0]
    for j in range(M):
        E.append(E[-1] + int(csq[j]))
    if mode == MODE_EARLY_STOP:
        N = 0
        for j in range(1, M + 1):
            # J_j > J_{j-1}  <=>  E_j * c(j-1) > E_{j-1} * c(j)   (c > 0); two separate fp64 products
            lhs = float(E[j]) * float(cost[j - 1])
            rhs = float(E[j - 1]) * float(cost[j])
            if lhs > rhs:
                N = j
            else:
                break
    elif mode == MODE_ARGMAX:
        if np.any(cost[:M + 1] <= 0):
            raise ValueError("argmax mode needs a positive step-time table")
        best, N = -1.0, 0
        for j in range(0, M + 1):
            Jj = float(E[j]) / float(cost[j])
            if Jj > best:
                best, N = Jj, j
    elif mode == MODE_TOP_M:
        N = M
    elif mode == MODE_THRESHOLD:
        windows = np.array([sum(1 for k in range(K) if S[i, k] >= threshold) for i in range(R)], dtype=np.int32)
        N = int(windows.sum())
        En = sum(int(Sq[i, k]) for i in range(R) for k in range(int(windows[i])))
        E_real = float(En) * (2.0 ** -Q)
        J = E_real / float(cost[N]) if cost[N] != 0 else (0.0 if E_real == 0 else math.inf)
        return dict(windows=windows, survival=S, N=N, E=E_real, J=J, Q=Q, order=(ci[:M], ck[:M]))
    else:
        raise ValueError("unknown mode")
    windows = np.zeros(R, dtype=np.int32)
    for j in range(N):
        windows[ci[j]] += 1
    E_real = float(E[N]) * (2.0 ** -Q)
    J = E_real / float(cost[N]) if cost[N] != 0 else (0.0 if E_real == 0 else math.inf)
    return dict(windows=windows, survival=S, N=N, E=E_real, J=J, Q=Q,
                order=(ci[:M], ck[:M]))
