"""Pins of the oracle's calibration metric (ECE of confidences against verify outcomes)."""
import json
import os

import numpy as np

from oracle import calibration as ocal

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_case():
    g = json.load(open(os.path.join(GOLD, "ece_case.json")))
    conf = np.array(g["conf"], dtype=np.float32)
    r = ocal.verify_ece(conf, g["cu_seqlens"], g["decided"], g["n_bins"])
    np.testing.assert_allclose(r["ece"], g["expected"]["ece"], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(r["n_obs"], g["expected"]["n_obs"])
    assert abs(r["ece_batch"] - g["expected"]["ece_batch"]) < 1e-15
    conf[1, 1] = g["variant"]["conf_1_1"]
    r = ocal.verify_ece(conf, g["cu_seqlens"], g["decided"], g["n_bins"])
    assert abs(r["ece"][1] - g["variant"]["ece_1"]) < 1e-15
    assert abs(r["ece_batch"] - g["variant"]["ece_batch"]) < 1e-15


def test_single_rejection_gives_its_confidence():
    for c in (0.0, 0.3, 0.7, 1.0):
        r = ocal.verify_ece(np.array([[c, 0.9]], np.float32), [0, 3], [0], 10)
        assert r["n_obs"][0] == 1
        assert abs(r["ece"][0] - np.float32(c)) < 1e-15


def test_perfect_calibration_is_zero():
    # confidence 1 and always accepted; and a bin whose mean outcome equals its mean confidence
    r = ocal.verify_ece(np.ones((3, 4), np.float32), [0, 5, 10, 15], [4, 4, 4], 10)
    assert np.all(r["ece"] == 0.0) and r["ece_batch"] == 0.0
    # four requests at confidence 0.75, window 1: three accepted, one rejected
    conf = np.full((4, 1), 0.75, np.float32)
    r = ocal.verify_ece(conf, [0, 2, 4, 6, 8], [1, 1, 1, 0], 10)
    assert r["ece_batch"] == 0.0


def test_undecided_positions_and_faults_carry_no_outcome():
    conf = np.full((2, 5), 0.5, np.float32)
    r = ocal.verify_ece(conf, [0, 6, 12], [2, -1], 4)
    assert list(r["n_obs"]) == [3, 0]
    assert r["ece"][1] == 0.0


def test_order_of_positions_within_a_bin_does_not_matter():
    rng = np.random.default_rng(3)
    c = rng.random(40)
    o = (rng.random(40) < c).astype(float)
    p = rng.permutation(40)
    assert abs(ocal.ece(c, o, 10) - ocal.ece(c[p], o[p], 10)) < 1e-15


def test_bin_edges():
    assert list(ocal.bin_index([0.0, 0.0999999, 0.1, 0.95, 1.0], 10)) == [0, 0, 1, 9, 9]
