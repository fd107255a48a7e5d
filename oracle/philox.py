"""Philox4x64-10 counter-based generator -- oracle side (test infrastructure).

Definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
Random Numbers: As Easy as 1, 2, 3", SC'11, section 3 (the Philox S-box built
from a 64x64->128 multiply, ten rounds, Weyl-sequence key schedule).

The source pages say only that rejection sampling draws a uniform per position
(DSpark study notes, section 1); they do not fix a generator. Both the oracle
and the HIP path implement this one counter-based generator independently, so
that every random decision is a pure function of (seed, round, request id,
position).

Pinned by: bit equality with numpy's own Philox bit generator (a separate
library implementation of the same published function) on many counters and
keys, and chi-square uniformity of the derived uniforms (tests/test_oracle_philox.py).
"""
import numpy as np

# Multipliers and key increments of Philox4x64 (SC'11, table of constants).
M0 = np.uint64(0xD2E7470EE14C6C93)
M1 = np.uint64(0xCA5A826395121157)
W0 = np.uint64(0x9E3779B97F4A7C15)
W1 = np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

# Word layout: counter = (round, request id, position, stream).
STREAM_VERIFY = 0
WORD_ACCEPT = 0      # uniform u_k compared with min(1, p/q)
WORD_SAMPLE = 1      # uniform u'_k for the residual (rejection at k) or bonus (k = n+1)
STREAM_DRAFT = 1     # the sampled Markov draft: word 0 draws the token of position d
WORD_DRAW = 0


def _mulhilo(a, b):
    """Full 64x64 -> 128-bit product of uint64 arrays, returned as (hi, lo)."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    a0, a1 = a & _LO32, a >> _S32
    b0, b1 = b & _LO32, b >> _S32
    p00 = a0 * b0
    p01 = a0 * b1
    p10 = a1 * b0
    p11 = a1 * b1
    mid = (p00 >> _S32) + (p01 & _LO32) + (p10 & _LO32)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    lo = a * b  # wraps mod 2^64
    return hi, lo


def philox4x64_10(ctr, key):
    """Philox4x64 with 10 rounds.

    ctr: uint64 array [..., 4]; key: uint64 array [..., 2] (broadcastable).
    Returns uint64 array [..., 4].
    """
    ctr = np.asarray(ctr, dtype=np.uint64)
    key = np.asarray(key, dtype=np.uint64)
    with np.errstate(over="ignore"):
        c0, c1, c2, c3 = (ctr[..., j].copy() for j in range(4))
        k0 = np.broadcast_to(key[..., 0], c0.shape).copy()
        k1 = np.broadcast_to(key[..., 1], c0.shape).copy()
        for r in range(10):
            if r > 0:
                k0 = k0 + W0
                k1 = k1 + W1
            hi0, lo0 = _mulhilo(M0, c0)
            hi1, lo1 = _mulhilo(M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1)


def to_unit_double(w):
    """Map a 64-bit word to a double in [0, 1): top 53 bits times 2^-53 (exact)."""
    w = np.asarray(w, dtype=np.uint64)
    return (w >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def verify_uniforms(seed, rnd, req_ids, kmax):
    """Uniforms for positions k = 1..kmax of each request.

    Returns (u, us): float64 arrays [len(req_ids), kmax]; column k-1 holds the
    accept uniform u_k and the sampling uniform u'_k for position k.
    """
    req_ids = np.asarray(req_ids, dtype=np.uint64)
    R = req_ids.shape[0]
    ctr = np.zeros((R, kmax, 4), dtype=np.uint64)
    ctr[..., 0] = np.uint64(rnd)
    ctr[..., 1] = req_ids[:, None]
    ctr[..., 2] = np.arange(1, kmax + 1, dtype=np.uint64)[None, :]
    ctr[..., 3] = np.uint64(STREAM_VERIFY)
    key = np.array([np.uint64(seed), np.uint64(0)], dtype=np.uint64)
    out = philox4x64_10(ctr, key)
    return to_unit_double(out[..., WORD_ACCEPT]), to_unit_double(out[..., WORD_SAMPLE])


def draft_uniforms(seed, rnd, req_ids, d):
    """Uniform of the sampled draft's token draw at position d (1-based) for each request.

    Counter (round, request id, d, STREAM_DRAFT), word 0; the verify step's
    counters use stream 0, so the two never share a block.
    """
    req_ids = np.asarray(req_ids, dtype=np.uint64)
    ctr = np.zeros((req_ids.shape[0], 4), dtype=np.uint64)
    ctr[:, 0] = np.uint64(rnd)
    ctr[:, 1] = req_ids
    ctr[:, 2] = np.uint64(d)
    ctr[:, 3] = np.uint64(STREAM_DRAFT)
    key = np.array([np.uint64(seed), np.uint64(0)], dtype=np.uint64)
    return to_unit_double(philox4x64_10(ctr, key)[:, WORD_DRAW])
