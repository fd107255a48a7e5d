"""Pins of the oracle's Markov-head greedy chain (DSpark study notes, section 4; PCTree article)."""
import json
import math
import os

import numpy as np
import pytest

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
        np.testing.assert_array_equal(np.argmax(z, -1), res["y"][:, d])
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
    np.testing.assert_array_equal(rep["y"][:, 2], np.argmax(z, -1))


# ---------------------------------------------------------------- sampled chain

def test_round_bf16_equals_integer_rounding_of_float32():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, 1.0, -1.0, 3.0, 1.00390625, 1.01171875])])
    got, _, _ = om.round_bf16(x.astype(np.float64))
    ref = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x)).astype(np.float64)
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_picks_nearest_enumerated_neighbour():
    """fp64 inputs (not representable in fp32) against every positive finite bf16 value."""
    allb = np.sort(workloads.bf16_bits_to_f32(np.arange(1, 0x7F80, dtype=np.uint16)).astype(np.float64))
    rng = np.random.default_rng(8)
    z = rng.uniform(0.01, 100.0, 20000) * (1 + 1e-12 * rng.standard_normal(20000))
    got, gap, ulp = om.round_bf16(z)
    j = np.searchsorted(allb, z)
    lo, hi = allb[j - 1], allb[j]
    dlo, dhi = z - lo, hi - z
    bits_lo = workloads.f32_to_bf16_bits(lo.astype(np.float32))
    even_lo = (bits_lo & 1) == 0
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(even_lo, lo, hi)))
    np.testing.assert_array_equal(got, want)
    np.testing.assert_allclose(gap, np.abs(dlo - dhi) / 2, rtol=1e-9, atol=1e-300)
    np.testing.assert_allclose(ulp, hi - lo, rtol=0)


def test_sampled_two_token_law_is_logistic():
    """V = 2, no Markov term: P(y = 1) = 1 / (1 + exp(-(l1 - l0) / T)) (closed form)."""
    for beta, T in ((0.5, 1.0), (-1.5, 0.7)):
        R = 400
        L = np.zeros((R, 1, 2), dtype=np.float32)
        L[:, 0, 1] = beta
        U = np.zeros((2, 32), dtype=np.float32)
        W = np.zeros((32, 2), dtype=np.float32)
        ones = 0
        N = 0
        for rnd in range(60):
            res = om.chain_sampled(L, U, W, np.zeros(R, dtype=np.int64), T, seed=11, rnd=rnd)
            ones += int(res["y"].sum())
            N += R
        a = 1.0 / (1.0 + math.exp(-beta / T))
        assert abs(ones / N - a) < 5 * math.sqrt(a * (1 - a) / N), (beta, T, ones / N, a)


def test_sampled_low_temperature_is_argmax_of_rounded_row():
    L, U, W, anchors = _small(R=8, B=3, V=300, r=32, seed=9)
    W = W * 300
    res = om.chain_sampled(L, U, W, anchors, 1e-3, seed=2)
    prev = anchors
    checked = 0
    for d in range(3):
        zh, _, _ = om.round_bf16(om.markov_logits(L[:, d], U, W, prev))
        top = -np.sort(-zh, axis=-1)
        for i in range(8):
            if top[i, 0] - top[i, 1] > 0.1:
                assert res["y"][i, d] == int(np.argmax(zh[i]))
                checked += 1
        prev = res["y"][:, d]
    assert checked >= 12


def test_sampled_replay_is_step_local():
    L, U, W, anchors = _small(R=4, B=4, V=120, r=32, seed=10)
    W = W * 300
    own = om.chain_sampled(L, U, W, anchors, 1.0, seed=5, rnd=3)
    forced = own["y"].copy()
    forced[:, 1] = (forced[:, 1] + 7) % 120
    rep = om.chain_sampled(L, U, W, anchors, 1.0, seed=5, rnd=3, forced=forced)
    np.testing.assert_array_equal(rep["y"][:, :2], own["y"][:, :2])
    np.testing.assert_array_equal(rep["zhat"][:, :2], own["zhat"][:, :2])
    z3 = om.round_bf16(om.markov_logits(L[:, 2], U, W, forced[:, 1]))[0]
    np.testing.assert_array_equal(rep["zhat"][:, 2], z3)
    np.testing.assert_allclose(np.exp(own["logq"]).sum() > 0, True)
    # logq_forced is the log-probability of the forced token under the step's rounded row
    s = z3 / 1.0
    lse = s.max(-1) + np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1))
    np.testing.assert_allclose(rep["logq_forced"][:, 2], s[np.arange(4), forced[:, 2]] - lse, rtol=1e-12)


def test_masked_logits_carry_no_mass():
    """A masked vocabulary entry (-inf base logit) rounds to -inf and is never drawn; with V = 3
    and token 2 masked the two remaining tokens keep the logistic law (closed form)."""
    got, gap, ulp = om.round_bf16(np.array([-np.inf, 1.5]))
    assert got[0] == -np.inf and gap[0] == np.inf and ulp[0] == 0.0 and got[1] == 1.5
    beta, T, R = 0.8, 1.0, 400
    L = np.zeros((R, 1, 3), dtype=np.float32)
    L[:, 0, 1] = beta
    L[:, 0, 2] = -np.inf
    U = np.zeros((3, 32), dtype=np.float32)
    W = np.zeros((32, 3), dtype=np.float32)
    ones, N = 0, 0
    for rnd in range(60):
        res = om.chain_sampled(L, U, W, np.zeros(R, dtype=np.int64), T, seed=12, rnd=rnd)
        assert not np.any(res["y"] == 2)
        assert np.all(res["round_tie"][..., 2] == False)  # noqa: E712
        ones += int(res["y"].sum())
        N += R
    a = 1.0 / (1.0 + math.exp(-beta / T))
    assert abs(ones / N - a) < 5 * math.sqrt(a * (1 - a) / N), (ones / N, a)
    # greedy chain: the masked token is never the argmax even when the rank term favours it
    Wg = np.zeros((32, 3), dtype=np.float32)
    Ug = np.ones((3, 32), dtype=np.float32)
    Wg[:, 2] = 10.0
    g = om.chain(L, Ug, Wg, np.zeros(R, dtype=np.int64))
    assert not np.any(g["y"] == 2)


def test_argmax_decides_on_fp64_values():
    """Two entries equal in fp32 but not in fp64: the argmax follows the fp64 values."""
    L = np.zeros((1, 1, 4), dtype=np.float64)
    L[0, 0, 1] = 1.0
    L[0, 0, 3] = 1.0 + 2.0 ** -40  # rounds to 1.0 in fp32
    assert np.float32(L[0, 0, 3]) == np.float32(1.0)
    U = np.zeros((4, 32))
    W = np.zeros((32, 4))
    res = om.chain(L, U, W, np.zeros(1, dtype=np.int64), want_margin=True)
    assert res["y"][0, 0] == 3
    assert res["margin"][0, 0] == 2.0 ** -40
    # exact ties go to the lowest id
    L[0, 0, 3] = 1.0
    assert om.chain(L, U, W, np.zeros(1, dtype=np.int64))["y"][0, 0] == 1


def _tie_rows(R, V, seed, T, frac=0.5):
    """Base logits sitting within ROUND_BAND of a bf16 rounding midpoint at a fraction of the
    entries (the rest ordinary), no Markov term: z = L exactly."""
    rng = np.random.default_rng(seed)
    vals = rng.normal(0.0, 2.0, (R, V))
    zh, _, ulp = om.round_bf16(vals)
    mid = zh + 0.5 * ulp * np.where(rng.random((R, V)) < 0.5, 1.0, -1.0)
    off = (rng.random((R, V)) - 0.5) * 1e-6 * np.maximum(1.0, np.abs(mid))
    near = rng.random((R, V)) < frac
    L = np.where(near, mid + off, vals)[:, None, :]
    return L


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_rounding_tie_bounds_hold_under_perturbation(T):
    """The bounds chain_sampled reports for rows whose near-midpoint entries may land one unit
    (plus the band) away, checked against explicit perturbations of those entries (random
    points and the corners of the allowed box): the CDF and L1 moves stay within tie_shift,
    and the drawn token's log-probability within tok_dev / T + log(1 / (1 - eps))."""
    R, V = 12, 48
    L = _tie_rows(R, V, 3, T)
    U, W = np.zeros((V, 32)), np.zeros((32, V))
    res = om.chain_sampled(L, U, W, np.zeros(R, dtype=np.int64), T, seed=4)
    assert res["round_tie"].sum() > R * V // 4
    z = L[:, 0, :]
    zh = res["zhat"][:, 0, :]
    tie = res["round_tie"][:, 0, :]
    _, _, ulp = om.round_bf16(z)
    dev = np.where(tie, ulp + om.ROUND_BAND * np.maximum(1.0, np.abs(z)), 0.0)
    rng = np.random.default_rng(9)
    worst = 0.0
    for i in range(R):
        x = int(res["y"][i, 0])
        q = np.exp(zh[i] / T - np.max(zh[i] / T))
        q /= q.sum()
        F = np.cumsum(q)
        for trial in range(200):
            s = rng.choice([-1.0, 1.0], V) if trial % 2 else rng.uniform(-1.0, 1.0, V)
            zp = zh[i] + s * dev[i]
            qp = np.exp(zp / T - np.max(zp / T))
            qp /= qp.sum()
            cdf_move = np.max(np.abs(np.cumsum(qp) - F))
            l1 = np.sum(np.abs(qp - q))
            assert cdf_move <= res["tie_shift"][i, 0] * (1 + 1e-9)
            assert l1 <= res["tie_shift"][i, 0] * (1 + 1e-9)
            lq_move = abs(np.log(qp[x]) - np.log(q[x]))
            assert lq_move <= res["tok_dev"][i, 0] / T - np.log1p(-res["eps"][i, 0]) + 1e-12
            worst = max(worst, cdf_move / res["tie_shift"][i, 0])
    assert worst > 0.2  # the bound is not vacuous on these rows


def test_verify_bands_keep_decisions_under_draft_rounding_ties():
    """A verify whose draft rows are perturbed within the rounding-tie box makes the oracle's
    decisions wherever the oracle's margin exceeds the band derived from eps and tok_dev
    (accept: ratio * expm1(eta); residual draw: 2 dq / sum(r)); many rounds of uniforms."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    from parity import rounding_bands
    from oracle import verify as ov
    T, R, K, V = 1.0, 6, 3, 40
    rng = np.random.default_rng(21)
    Ld = np.concatenate([_tie_rows(R, V, 30 + k, T, frac=0.1) for k in range(K)], axis=1)  # [R, K, V]
    U, W = np.zeros((V, 32)), np.zeros((32, V))
    # per position one sampled chain step over that position's rows (no Markov term)
    od = [om.chain_sampled(Ld[:, k:k + 1], U, W, np.zeros(R, dtype=np.int64), T, seed=5) for k in range(K)]
    zhat = np.concatenate([o["zhat"] for o in od], axis=1)
    x = np.concatenate([o["y"] for o in od], axis=1)
    eps = np.concatenate([o["eps"] for o in od], axis=1)
    tok_dev = np.concatenate([o["tok_dev"] for o in od], axis=1)
    tie = np.concatenate([o["round_tie"] for o in od], axis=1)
    _, _, ulp = om.round_bf16(Ld)
    dev = np.where(tie, ulp + om.ROUND_BAND * np.maximum(1.0, np.abs(Ld)), 0.0)
    # target rows close to the draft's so that acceptance is frequent and residuals small
    tgt = np.concatenate([np.concatenate([zhat[i] + rng.normal(0, 0.8, (K, V)), rng.normal(0, 2, (1, V))])
                          for i in range(R)])
    cu = np.arange(R + 1) * (K + 1)
    checked, resid = 0, 0
    for trial in range(6):
        s = rng.choice([-1.0, 1.0], zhat.shape) if trial % 2 else rng.uniform(-1.0, 1.0, zhat.shape)
        zp = zhat + s * dev
        for rnd in range(40):
            own = ov.verify_chain(tgt, cu, zhat, x, T, seed=1, rnd=rnd)
            alt = ov.verify_chain(tgt, cu, zp, x, T, seed=1, rnd=rnd)
            acc_band, _ = rounding_bands(own, eps, tok_dev, T)
            for i in range(R):
                a = int(own["accepted_len"][i])
                decided = range(min(K, a + 1))
                if all(own["accept_margin"][i, k] >= acc_band[i, k] for k in decided):
                    assert alt["accepted_len"][i] == a
                    _, smp_band = rounding_bands(own, eps, tok_dev, T)
                    if own["sample_margin"][i] >= smp_band[i]:
                        assert alt["out_tokens"][i, a] == own["out_tokens"][i, a]
                        checked += 1
                        resid += int(own["resid_mass"][i] > 0)
    print("checked", checked, "residual draws", resid)
    assert checked > 500 and resid > 100
