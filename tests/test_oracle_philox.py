"""Pins of the oracle's Philox4x64-10 (Salmon et al., SC'11) against an independent library."""
import numpy as np
import pytest

from oracle import philox


def _numpy_block(ctr, key):
    # numpy's Philox increments the counter before producing its first block
    g = np.random.Philox(key=[int(key[0]), int(key[1])],
                         counter=[int(ctr[0]) - 1, int(ctr[1]), int(ctr[2]), int(ctr[3])])
    return np.array(g.random_raw(4), dtype=np.uint64)


def test_block_matches_numpy_philox():
    rng = np.random.Generator(np.random.PCG64(7))
    ctrs = rng.integers(1, 2**63, size=(200, 4), dtype=np.uint64)
    keys = rng.integers(0, 2**63, size=(200, 2), dtype=np.uint64)
    ctrs[:20, 1:] = 0  # small counters like the verify layout uses
    ctrs[:20, 0] = np.arange(1, 21)
    ours = philox.philox4x64_10(ctrs, keys)
    for j in range(ctrs.shape[0]):
        np.testing.assert_array_equal(ours[j], _numpy_block(ctrs[j], keys[j]))


def test_high_bits_paths_match_numpy():
    # counters and keys with the top bit set exercise the 128-bit product carries
    ctr = np.array([2**64 - 5, 2**64 - 1, 2**63 + 12345, 2**64 - 2], dtype=np.uint64)
    key = np.array([2**64 - 1, 2**64 - 3], dtype=np.uint64)
    np.testing.assert_array_equal(philox.philox4x64_10(ctr, key), _numpy_block(ctr, key))


def test_unit_double_range_and_exactness():
    w = np.array([0, 1 << 11, 2**64 - 1], dtype=np.uint64)
    u = philox.to_unit_double(w)
    assert u[0] == 0.0 and u[1] == 2.0 ** -53 and u[2] == 1.0 - 2.0 ** -53


def test_uniforms_chi_square():
    from scipy import stats
    u, us = philox.verify_uniforms(seed=0, rnd=3, req_ids=np.arange(20000), kmax=50)
    for arr in (u, us):
        counts, _ = np.histogram(arr.ravel(), bins=1000, range=(0.0, 1.0))
        chi2 = ((counts - arr.size / 1000) ** 2 / (arr.size / 1000)).sum()
        assert stats.chi2.sf(chi2, 999) > 1e-4
    # accept and sample words are uncorrelated
    assert abs(np.corrcoef(u.ravel(), us.ravel())[0, 1]) < 5e-3


def test_uniforms_depend_on_every_counter_field():
    base = philox.verify_uniforms(1, 2, [3], 4)[0]
    assert not np.array_equal(base, philox.verify_uniforms(9, 2, [3], 4)[0])
    assert not np.array_equal(base, philox.verify_uniforms(1, 5, [3], 4)[0])
    assert not np.array_equal(base, philox.verify_uniforms(1, 2, [4], 4)[0])
    assert len(np.unique(base)) == 4
    np.testing.assert_array_equal(base, philox.verify_uniforms(1, 2, [3], 4)[0])
