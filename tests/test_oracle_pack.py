"""Pins of the oracle's ragged pack (SGLang article, "Ragged verify")."""
import numpy as np

from oracle import pack as op


def test_cumsum_and_row_maps():
    rng = np.random.Generator(np.random.PCG64(1))
    for _ in range(20):
        R, K = int(rng.integers(1, 50)), int(rng.integers(1, 17))
        w = rng.integers(0, K + 1, size=R)
        anchors = rng.integers(0, 1000, size=R)
        drafts = rng.integers(0, 1000, size=(R, K))
        r = op.pack_ragged(w, anchors, drafts)
        np.testing.assert_array_equal(r["cu_seqlens"], np.concatenate([[0], np.cumsum(w + 1)]))
        assert r["total"] == R + w.sum() == r["tokens"].shape[0]
        pairs = set(zip(r["row_req"].tolist(), r["row_pos"].tolist()))
        assert pairs == {(i, k) for i in range(R) for k in range(w[i] + 1)}
        for j in range(r["total"]):
            i, k = r["row_req"][j], r["row_pos"][j]
            assert r["tokens"][j] == (anchors[i] if k == 0 else drafts[i, k - 1])


def test_hand_fixture_and_tiers():
    r = op.pack_ragged([2, 0, 3], [10, 20, 30], [[1, 2, 3], [4, 5, 6], [7, 8, 9]],
                       tiers=[4, 8, 16])
    assert r["cu_seqlens"].tolist() == [0, 3, 4, 8]
    assert r["tokens"].tolist() == [10, 1, 2, 20, 30, 7, 8, 9]
    assert r["row_req"].tolist() == [0, 0, 0, 1, 2, 2, 2, 2]
    assert r["row_pos"].tolist() == [0, 1, 2, 0, 0, 1, 2, 3]
    assert r["total"] == 8 and r["tier"] == 8
    assert op.pack_ragged([5], [0], [[1] * 5], tiers=[4])["tier"] == -1
    assert op.pack_ragged([1], [0], [[1]])["tier"] == 2
