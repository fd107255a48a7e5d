"""Pins of the oracle's Markov-head greedy chain (DSpark study notes, section 4; PCTree article)."""
import json
import math
import os

import numpy as np

import workloads
from oracle import markov as om

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _small(R=6, B=5, V=300, r=32, seed=1):
    c = workloads.markov_case(R, B, V, rank=r, seed=seed)
    return (workloads.bf16_bits_to_f32(c["L"]), workloads.bf16_bits_to_f32(c["U"]),
            workloads.bf16_bits_to_f32(c["W"]), c["anchors"])


def test_zero_markov_term_is_plain_argmax():
    L, U, W, anchors = _small()
    res = om.chain(L, U, np.zeros_like(W), anchors)
    np.testing.assert_array_equal(res["y"], np.argmax(L, axis=-1))


def test_rank_term_matches_independent_dot_products():
    L, U, W, anchors = _small(R=3, B=2, V=64, r=32)
    prev = np.array([5, 17, 63])
    z = om.markov_logits(L[:, 0], U, W, prev)
    for i in range(3):
        for v in (0, 7, 31, 63):
            ref = float(L[i, 0, v]) + math.fsum(float(U[prev[i], j]) * float(W[j, v]) for j in range(32))
            assert abs(z[i, v] - ref) < 1e-12


def test_chain_conditions_on_previous_choice():
    """Step d uses y_{d-1}: re-running one step from the chosen tokens reproduces y_d."""
    L, U, W, anchors = _small(R=4, B=6, V=200, r=32, seed=3)
    W = W * 400  # make the Markov term matter
    res = om.chain(L, U, W, anchors)
    prev = anchors
    for d in range(6):
        z = om.markov_logits(L[:, d], U, W, prev)
        np.testing.assert_array_equal(np.argmax(z.astype(np.float32), -1), res["y"][:, d])
        prev = res["y"][:, d]
    # and differs from conditioning on the anchor at every step
    z0 = om.markov_logits(L[:, 3], U, W, anchors)
    assert not np.array_equal(np.argmax(z0, -1), res["y"][:, 3])


def test_logq_is_normalised_log_probability():
    L, U, W, anchors = _small()
    res = om.chain(L, U, W, anchors)
    assert np.all(res["logq"] <= 0)
    prev = anchors
    for d in range(L.shape[1]):
        z = om.markov_logits(L[:, d], U, W, prev)
        p = np.exp(z - z.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        np.testing.assert_allclose(np.exp(res["logq"][:, d]), p[np.arange(len(prev)), res["y"][:, d]],
                                   rtol=1e-12)
        prev = res["y"][:, d]


def test_of_course_fixture():
    g = json.load(open(os.path.join(GOLD, "of_course_markov.json")))
    tok = g["tokens"]
    inv = {v: k for k, v in tok.items()}
    L = np.array(g["L"], dtype=np.float32)[None]
    U = np.array(g["U"], dtype=np.float32)
    W = np.array(g["W"], dtype=np.float32)
    a = np.array([tok["anchor"]])
    plain = om.chain(L, U, np.zeros_like(W), a)["y"][0]
    assert [inv[int(v)] for v in plain] == g["expected_without_markov"]
    boosted = om.chain(L, U, W, a)["y"][0]
    assert [inv[int(v)] for v in boosted] == g["expected_with_markov"]


def test_forced_replay_is_step_local():
    L, U, W, anchors = _small(R=3, B=4, V=100, r=32, seed=4)
    W = W * 300
    own = om.chain(L, U, W, anchors)["y"]
    forced = own.copy()
    forced[:, 1] = (forced[:, 1] + 1) % 100
    rep = om.chain(L, U, W, anchors, forced=forced)
    np.testing.assert_array_equal(rep["y"][:, :2], own[:, :2])
    z = om.markov_logits(L[:, 2], U, W, forced[:, 1])
    np.testing.assert_array_equal(rep["y"][:, 2], np.argmax(z.astype(np.float32), -1))
