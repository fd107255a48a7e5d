"""Pins of the oracle's confidence head with sequential temperature scaling (DSpark study
notes, section 5.1; SGLang article, STS)."""
import math

import numpy as np

from oracle import confidence as oc


def test_unit_weight_picks_one_coordinate():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((3, 4, 16))
    w = np.zeros(16)
    w[5] = 1.0
    T = np.array([1.0, 0.5, 2.0, 4.0])
    c = oc.confidence_head(h, w, 0.25, T)
    for i in range(3):
        for k in range(4):
            assert abs(c[i, k] - 1.0 / (1.0 + math.exp(-(h[i, k, 5] + 0.25) / T[k]))) < 1e-15


def test_zero_logit_is_one_half_and_symmetry():
    h = np.zeros((2, 3, 8))
    assert np.all(oc.confidence_head(h, np.ones(8), 0.0) == 0.5)
    rng = np.random.default_rng(2)
    h = rng.standard_normal((2, 3, 8))
    w = rng.standard_normal(8)
    a = oc.confidence_head(h, w, 0.3)
    b = oc.confidence_head(-h, w, -0.3)
    np.testing.assert_allclose(a + b, 1.0, rtol=0, atol=1e-15)


def test_temperature_flattens_towards_one_half():
    rng = np.random.default_rng(3)
    h = rng.standard_normal((2, 5, 32))
    w = rng.standard_normal(32)
    prev = None
    for T in (0.5, 1.0, 4.0, 64.0):
        c = oc.confidence_head(h, w, 0.1, np.full(5, T))
        d = np.abs(c - 0.5)
        if prev is not None:
            assert np.all(d <= prev + 1e-15)
        prev = d
    assert np.all(prev < 0.1)
