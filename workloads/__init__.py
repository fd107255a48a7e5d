"""Seeded synthetic workloads shared by the oracle checks, the GPU tests and the benchmark.

This module only draws random inputs; it computes nothing the method computes
(no softmax, no acceptance test, no scheduling, no Markov scores). Every array is
produced by numpy's PCG64 from a fixed seed, so both sides of a parity check see
identical bytes.

Shapes follow the workloads the source pages describe: block 7 offline and
block 16 (DSpark study notes, sections 7-8; PCTree article), Qwen3's 151,936
vocabulary and DeepSeek-V4's 129,280, concurrency up to 256 with mixed easy and
hard streams (SGLang article). The public benchmarks those pages evaluate on are
not used; these synthetic logits stand in for them.

Recipes (N(m, s) = normal with mean m and standard deviation s):

* tiny verify: R=4, K=7, V=1024, fp32 target t ~ N(0, 2) of shape [R, K+1, V];
  draft d_{i,k} = t_{i,k-1} + N(0, 0.5); confidence sigmoid(N(1, 1)).
* dense-vocab verify: R=64, K=7, V=151,936, bf16; t ~ N(0, 3) plus 8 on an
  i.i.d. 1% of entries; d_{i,k} = t_{i,k-1} + sigma * eps with eps ~ N(0, 1) and
  sigma from ``calibration.json`` (chosen by a committed oracle script so the
  mean one-token acceptance is about 0.8).
* scheduled ragged verify: R=256, K=16, V=151,936, bf16; t as the dense-vocab verify; a noise
  scale sigma_i ~ U(0.2, 2.0) per request (easy and hard streams);
  d = t + sigma_i * eps; confidence c_{i,k} = sigmoid(4 - 8 TV_{i,k} + 0.25 eta),
  eta ~ N(0, 1), a logistic model of the draft-target gap measured as the total-variation
  distance between the target and draft distributions of the position (TV from
  scheduled_tv.json, written by the oracle's calibration script: this module computes no
  softmax); additive cost table c(n) = 1.0 + 0.05 n.
* Markov chain: R=256, B=16, V=151,936, rank 256; L ~ N(0, 3) bf16;
  U [V, r], W [r, V] ~ N(0, 0.02) bf16; anchors uniform over the vocabulary.
* RNN sequential head: the Markov case's L, anchors and second factor (as W_o); backbone
  states h [R, B, H] ~ N(0, 1) bf16; A [r, r] ~ N(0, 1/sqrt(r)), E [V, r] ~ N(0, 0.5),
  G [H, r] ~ N(0, 0.5/sqrt(H)) (stored transposed), bias ~ N(0, 0.1).
* PCTree + tree verify: R=128, D=16, V=129,280, rank 256, k=4, F=16, N=64;
  L, U, W as the Markov chain; target logits for the root and each tree node ~ N(0, 3) bf16.

* draft -> schedule -> pack -> verify cycle: the Markov-chain inputs (L, U, W,
  anchors) draft K positions per request; a noise scale sigma_i ~ U(0.2, 2.0)
  per request sets both the confidence sigmoid(4 - 2.5 sigma_i + 0.25 eta) and
  the target row that predicts draft position k, t_{i,k-1} = L_{i,k-1} +
  sigma_i * eps (t_{i,K} ~ N(0, 3)); the target rows are laid out in packed
  order for given windows (standing in for the target forward over the packed
  buffer); cost c(n) = 1.0 + 0.05 n.

* confidence head (the cycle builds its hidden states so that the head reproduces
  the cycle's confidences; see cycle_head_inputs): hidden states h [R, K, H] ~ N(0, 1) bf16, weights w [H] ~
  N(0, 1) / sqrt(H) bf16 (logits of unit scale), bias 1.5, sequential
  temperatures T_k = 1 + 0.05 k.

Draft tokens x_{i,k} are the synthetic draft model's samples from softmax(d/T)
(Gumbel-max with this module's own noise), or argmax d when T = 0.
"""
import hashlib
import json
import os

import numpy as np

V_QWEN3 = 151936
V_DSV4 = 129280

_HERE = os.path.dirname(os.path.abspath(__file__))


def f32_to_bf16_bits(x):
    """Round float32 to bfloat16 (round to nearest even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact float32 values of bfloat16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def calibration():
    with open(os.path.join(_HERE, "calibration.json")) as f:
        return json.load(f)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _store(x32, dtype):
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def values(arr, dtype):
    """Float32 view of stored logits (bf16 bits are widened exactly)."""
    return bf16_bits_to_f32(arr) if dtype == "bf16" else np.asarray(arr, np.float32)


def _draw_tokens(rng, d32, temperature):
    if temperature == 0.0:
        return np.argmax(d32, axis=-1).astype(np.int32)
    g = -np.log(-np.log(rng.random(d32.shape, dtype=np.float64).clip(1e-300, None)))
    return np.argmax(d32.astype(np.float64) / temperature + g, axis=-1).astype(np.int32)


def verify_case(R, K, V, dtype="bf16", seed=0, t_sigma=3.0, boost_p=0.0, boost=8.0,
                d_sigma=0.5, temperature=1.0):
    """Dense target [R, K+1, V] and draft [R, K, V] logits plus draft tokens [R, K].

    d_sigma: scalar or per-request array of draft noise scales.
    """
    rng = _rng(seed)
    d_sig = np.broadcast_to(np.asarray(d_sigma, dtype=np.float32), (R,))
    t_store = np.empty((R, K + 1, V), dtype=np.uint16 if dtype == "bf16" else np.float32)
    d_store = np.empty((R, K, V), dtype=t_store.dtype)
    x = np.empty((R, K), dtype=np.int32)
    for i in range(R):
        t = rng.standard_normal((K + 1, V), dtype=np.float32) * np.float32(t_sigma)
        if boost_p > 0:
            t += np.float32(boost) * (rng.random((K + 1, V), dtype=np.float32) < boost_p)
        t_store[i] = _store(t, dtype)
        tv = values(t_store[i], dtype)
        eps = rng.standard_normal((K, V), dtype=np.float32)
        d_store[i] = _store(tv[:K] + d_sig[i] * eps, dtype)
        x[i] = _draw_tokens(rng, values(d_store[i], dtype), temperature)
    return dict(t=t_store, d=d_store, x=x, dtype=dtype, R=R, K=K, V=V, temperature=temperature)


def confidences(rng, R, K, mean=1.0, std=1.0):
    return (1.0 / (1.0 + np.exp(-(mean + std * rng.standard_normal((R, K)))))).astype(np.float32)


def tiny_verify():
    """Tiny verify: 4 requests, K=7, V=1024, fp32, Philox seed 0."""
    c = verify_case(4, 7, 1024, dtype="f32", seed=1001, t_sigma=2.0, d_sigma=0.5)
    c["conf"] = confidences(_rng(2001), 4, 7)
    c["anchors"] = _rng(3001).integers(0, 1024, size=4).astype(np.int32)
    c["cost"] = 1.0 + 0.05 * np.arange(4 * 7 + 1, dtype=np.float64)
    return c


def dense_verify(sigma=None):
    """Dense-vocab verify: 64 requests, K=7, V=151,936, bf16, full-block windows."""
    if sigma is None:
        sigma = calibration()["dense_verify_sigma"]
    c = verify_case(64, 7, V_QWEN3, dtype="bf16", seed=1002, t_sigma=3.0, boost_p=0.01,
                    boost=8.0, d_sigma=sigma)
    c["conf"] = confidences(_rng(2002), 64, 7)
    c["anchors"] = _rng(3002).integers(0, V_QWEN3, size=64).astype(np.int32)
    # flat step-time table: every candidate with nonzero survival raises throughput,
    # so the scheduler returns full-block windows
    c["cost"] = np.ones(64 * 7 + 1, dtype=np.float64)
    c["sigma"] = sigma
    return c


def scheduled_verify_inputs(R=256, K=16, V=V_QWEN3):
    """Cost table, per-request noise scales, confidence noise and anchors of the scheduled
    verify (no logits, no confidences)."""
    rng = _rng(2003)
    sig = rng.uniform(0.2, 2.0, size=R).astype(np.float32)
    eta = rng.standard_normal((R, K))
    cost = 1.0 + 0.05 * np.arange(R * K + 1, dtype=np.float64)
    return dict(cost=cost, sigma_i=sig, eta=eta,
                anchors=_rng(3003).integers(0, V, size=R).astype(np.int32))


def scheduled_logits_hash(c):
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(c["t"]).tobytes())
    h.update(np.ascontiguousarray(c["d"]).tobytes())
    return h.hexdigest()[:16]


def scheduled_confidences(eta, tv):
    """c_{i,k} = sigmoid(4 - 8 TV_{i,k} + 0.25 eta_{i,k}) as float32."""
    z = 4.0 - 8.0 * np.asarray(tv, dtype=np.float64) + 0.25 * eta
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def scheduled_verify_schedule_inputs(R=256, K=16, V=V_QWEN3):
    """The scheduled verify's scheduler inputs (confidences from the stored TV table, cost
    table, anchors) without generating its logits; the full loader checks the table's hash."""
    s = scheduled_verify_inputs(R, K, V)
    with open(os.path.join(_HERE, "scheduled_tv.json")) as f:
        tvj = json.load(f)
    assert (tvj["R"], tvj["K"]) == (R, K)
    s["tv"] = np.asarray(tvj["tv"], dtype=np.float64)
    s["conf"] = scheduled_confidences(s["eta"], s["tv"])
    return s


def scheduled_verify(R=256, K=16, V=V_QWEN3, with_conf=True):
    """Confidence-scheduled ragged verify: mixed easy/hard streams, additive cost table.

    The confidences need the total-variation distances of the logits, which this module does
    not compute: they are read from scheduled_tv.json (written by the oracle's calibration
    script for exactly these logits; the stored hash is checked)."""
    s = scheduled_verify_inputs(R, K, V)
    c = verify_case(R, K, V, dtype="bf16", seed=1003, t_sigma=3.0, boost_p=0.01, boost=8.0,
                    d_sigma=s["sigma_i"])
    c.update(s)
    if with_conf:
        with open(os.path.join(_HERE, "scheduled_tv.json")) as f:
            tvj = json.load(f)
        assert (tvj["R"], tvj["K"]) == (R, K) and tvj["logits_sha256"] == scheduled_logits_hash(c), \
            "scheduled_tv.json was computed for other logits: rerun python -m oracle.calibrate_scheduled_verify"
        c["tv"] = np.asarray(tvj["tv"], dtype=np.float64)
        c["conf"] = scheduled_confidences(s["eta"], c["tv"])
    return c


def markov_case(R, B, V, rank=256, seed=1004, l_sigma=3.0, w_sigma=0.02):
    """Base logits L [R, B, V], factors U [V, r], W [r, V] (bf16 bits) and anchors [R]."""
    rng = _rng(seed)
    L = np.empty((R, B, V), dtype=np.uint16)
    for i in range(R):
        L[i] = f32_to_bf16_bits(rng.standard_normal((B, V), dtype=np.float32) * np.float32(l_sigma))
    U = f32_to_bf16_bits(rng.standard_normal((V, rank), dtype=np.float32) * np.float32(w_sigma))
    W = f32_to_bf16_bits(rng.standard_normal((rank, V), dtype=np.float32) * np.float32(w_sigma))
    anchors = rng.integers(0, V, size=R).astype(np.int32)
    return dict(L=L, U=U, W=W, anchors=anchors, R=R, B=B, V=V, rank=rank)


def rnn_case(R, B, V, rank=256, H=4096, seed=1007, wo_scale=1.0):
    """Inputs of the RNN sequential head: the Markov case's base logits L, anchors and
    second factor (as W_o, times wo_scale), plus backbone states h [R, B, H] ~ N(0, 1),
    memo-to-memo A [r, r] ~ N(0, 1/sqrt(r)), token table E [V, r] ~ N(0, 0.5), state
    projection G [H, r] ~ N(0, 0.5/sqrt(H)) stored transposed (Gt [r, H]) and a bias
    [r] ~ N(0, 0.1); all bf16 bits except the float32 bias."""
    c = markov_case(R, B, V, rank=rank, seed=seed)
    rng = _rng(seed + 3)
    Wo = bf16_bits_to_f32(c.pop("W")) * np.float32(wo_scale)
    c.pop("U")
    h = np.empty((R, B, H), dtype=np.uint16)
    for i in range(R):
        h[i] = f32_to_bf16_bits(rng.standard_normal((B, H), dtype=np.float32))
    c.update(Wo=f32_to_bf16_bits(Wo), h=h, H=H,
             A=f32_to_bf16_bits(rng.standard_normal((rank, rank), dtype=np.float32) / np.float32(np.sqrt(rank))),
             E=f32_to_bf16_bits(rng.standard_normal((V, rank), dtype=np.float32) * np.float32(0.5)),
             Gt=f32_to_bf16_bits(rng.standard_normal((rank, H), dtype=np.float32) * np.float32(0.5 / np.sqrt(H))),
             bias=(rng.standard_normal(rank) * 0.1).astype(np.float32))
    return c


def markov_chain():
    """Markov chain: 256 requests, 16 steps, V=151,936, rank 256."""
    return markov_case(256, 16, V_QWEN3, 256, seed=1004)


def tree_target(R, n_rows, V, seed, sigma=3.0):
    """Target logits [R, n_rows, V] bf16 for the root and each tree node."""
    rng = _rng(seed)
    out = np.empty((R, n_rows, V), dtype=np.uint16)
    for i in range(R):
        out[i] = f32_to_bf16_bits(rng.standard_normal((n_rows, V), dtype=np.float32) * np.float32(sigma))
    return out


def pctree():
    """PCTree + tree verify: 128 requests, depth 16, V=129,280, k=4, F=16, N=64."""
    c = markov_case(128, 16, V_DSV4, 256, seed=1005)
    c.update(topk=4, frontier=16, topN=64)
    c["target"] = tree_target(128, 65, V_DSV4, seed=2005)
    return c


def cycle_case(R, K, V, rank, seed):
    """Inputs of the draft -> schedule -> pack -> verify cycle (see the module docstring)."""
    c = markov_case(R, K, V, rank=rank, seed=seed)
    rng = _rng(seed + 7)
    sig = rng.uniform(0.2, 2.0, size=R).astype(np.float32)
    eta = rng.standard_normal((R, K))
    logit = 4.0 - 2.5 * sig[:, None] + 0.25 * eta
    c["conf"] = (1.0 / (1.0 + np.exp(-logit))).astype(np.float32)
    c["cost"] = 1.0 + 0.05 * np.arange(R * K + 1, dtype=np.float64)
    c["sigma"] = sig
    c["K"] = K
    c["target_seed"] = seed + 11
    c["logit"] = logit
    return c


def cycle_head_inputs(c, H=4096):
    """Hidden states and head weights for the cycle whose confidence head reproduces the
    cycle's confidences: h_{i,k} carries (T_k * logit_{i,k} - bias) / |w|^2 along w plus
    Gaussian noise orthogonal to w, so sigmoid((w . h + bias) / T_k) ~ conf_{i,k} (up to the
    bf16 rounding of h)."""
    rng = _rng(c["target_seed"] + 1)
    R, K = c["R"], c["K"]
    w = f32_to_bf16_bits(rng.standard_normal(H, dtype=np.float32) / np.float32(np.sqrt(H)))
    w64 = bf16_bits_to_f32(w).astype(np.float64)
    temps = (1.0 + 0.05 * np.arange(K)).astype(np.float32)
    bias = 1.5
    along = (temps[None, :].astype(np.float64) * c["logit"] - bias) / float(w64 @ w64)
    h = np.empty((R, K, H), dtype=np.uint16)
    for i in range(R):
        e = rng.standard_normal((K, H))
        e -= np.outer(e @ w64, w64) / float(w64 @ w64)
        h[i] = f32_to_bf16_bits((along[i][:, None] * w64[None, :] + e).astype(np.float32))
    return dict(h=h, w=w, bias=bias, temps=temps, H=H)


def cycle_target(c, windows):
    """Packed target rows (bf16 bits) for the given windows: request i owns rows for positions
    0..windows[i]; the row of position k < K is L_{i,k} + sigma_i * eps, that of position K is
    N(0, 3). Rows are drawn in packed order from one generator, so they depend only on the
    windows and the case."""
    rng = _rng(c["target_seed"])
    L = c["L"]
    R, K, V = c["R"], c["K"], c["V"]
    rows = []
    for i in range(R):
        for k in range(int(windows[i]) + 1):
            eps = rng.standard_normal(V, dtype=np.float32)
            if k < K:
                rows.append(f32_to_bf16_bits(bf16_bits_to_f32(L[i, k]) + c["sigma"][i] * eps))
            else:
                rows.append(f32_to_bf16_bits(np.float32(3.0) * eps))
    return np.stack(rows)


def confidence_case(R, K, H, seed):
    """Inputs of the confidence head (see the module docstring)."""
    rng = _rng(seed)
    h = f32_to_bf16_bits(rng.standard_normal((R, K, H), dtype=np.float32))
    w = f32_to_bf16_bits(rng.standard_normal(H, dtype=np.float32) / np.float32(np.sqrt(H)))
    temps = (1.0 + 0.05 * np.arange(K)).astype(np.float32)
    return dict(h=h, w=w, bias=1.5, temps=temps, R=R, K=K, H=H)
