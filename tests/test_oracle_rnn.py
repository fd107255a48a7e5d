"""Pins of the oracle's RNN sequential head (DSpark study notes, section 4)."""
import json
import math
import os

import numpy as np

import workloads
from oracle import markov as om
from oracle import rnn as orn

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _case(R=5, B=4, V=300, r=32, H=48, seed=1, scale=1.0):
    rng = np.random.default_rng(seed)
    c = workloads.markov_case(R, B, V, rank=r, seed=seed)
    L = workloads.bf16_bits_to_f32(c["L"]).astype(np.float64)
    Wo = workloads.bf16_bits_to_f32(c["W"]).astype(np.float64) * 100 * scale
    h = rng.normal(0, 1, (R, B, H))
    A = rng.normal(0, 0.3, (r, r))
    E = rng.normal(0, 0.5, (V, r))
    G = rng.normal(0, 0.2, (H, r))
    b = rng.normal(0, 0.1, r)
    return L, h, A, E, G, b, Wo, c["anchors"]


def test_no_recurrence_no_state_is_a_markov_head():
    """A = 0, G = 0: the memo of step d is tanh(E[y_{d-1}] + b) rounded to bf16, so the head is
    the Markov head whose first factor is that table."""
    L, h, A, E, G, b, Wo, a = _case(seed=2)
    res = orn.rnn_chain(L, h, np.zeros_like(A), E, np.zeros_like(G), b, Wo, a)
    U = om.round_bf16(np.tanh(E + b))[0]
    ch = om.chain(L, U, Wo, a)
    np.testing.assert_array_equal(res["y"], ch["y"])
    np.testing.assert_allclose(res["logq"], ch["logq"], rtol=1e-12, atol=1e-12)


def test_zero_projection_is_argmax_of_base_logits():
    L, h, A, E, G, b, Wo, a = _case(seed=3)
    res = orn.rnn_chain(L, h, A, E, G, b, np.zeros_like(Wo), a)
    np.testing.assert_array_equal(res["y"], np.argmax(L, axis=-1))


def test_memory_fixture():
    g = json.load(open(os.path.join(GOLD, "rnn_memory.json")))
    L = np.array(g["L"], dtype=np.float64)
    R, B, V = L.shape
    r = g["rank"]
    E, A, Wo = (np.array(g[k], dtype=np.float64) for k in ("E", "A", "Wo"))
    h = np.zeros((R, B, 1))
    G = np.zeros((1, r))
    a = np.full(R, g["anchor"])
    res = orn.rnn_chain(L, h, A, E, G, None, Wo, a)
    assert res["y"].tolist() == g["expected"]
    res0 = orn.rnn_chain(L, h, np.zeros_like(A), E, G, None, Wo, a)
    assert res0["y"].tolist() == g["expected_without_carry"]


def test_recurrence_step_by_step():
    """Tiny case against a scalar evaluation of the update, one entry at a time."""
    L, h, A, E, G, b, Wo, a = _case(R=2, B=3, V=40, r=4, H=3, seed=4)
    res = orn.rnn_chain(L, h, A, E, G, b, Wo, a)
    for i in range(2):
        s = [0.0] * 4
        prev = int(a[i])
        for d in range(3):
            s = [math.tanh(math.fsum([s[k] * A[k, j] for k in range(4)] + [E[prev, j], b[j]] +
                                     [h[i, d, q] * G[q, j] for q in range(3)])) for j in range(4)]
            np.testing.assert_allclose(res["memo"][i, d], s, rtol=1e-13, atol=1e-15)
            sb = om.round_bf16(np.array(s))[0]
            z = [L[i, d, v] + math.fsum(sb[j] * Wo[j, v] for j in range(4)) for v in range(40)]
            assert res["y"][i, d] == int(np.argmax(z))
            prev = int(res["y"][i, d])


def test_forced_replay_conditions_on_the_given_tokens():
    L, h, A, E, G, b, Wo, a = _case(seed=5, scale=3.0)
    own = orn.rnn_chain(L, h, A, E, G, b, Wo, a)
    forced = own["y"].copy()
    forced[:, 1] = (forced[:, 1] + 11) % L.shape[2]
    rep = orn.rnn_chain(L, h, A, E, G, b, Wo, a, forced=forced)
    np.testing.assert_array_equal(rep["y"][:, :2], own["y"][:, :2])
    assert not np.array_equal(rep["memo"][:, 2], own["memo"][:, 2])
