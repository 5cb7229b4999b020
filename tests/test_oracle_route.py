"""Pins for the oracle's router and expert grouping (CPU only)."""
import math

import numpy as np
import pytest

import bruteforce
import oracle


def test_route_matches_full_sort():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((50, 256)).astype(np.float32)
    ids, w = oracle.route(lg, 6)
    ids2, w2 = bruteforce.route(lg, 6)
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=2 ** -23, atol=0)


def test_route_ties_go_to_lower_index():
    lg = np.array([[0.5, 2.0, 2.0, -1.0, 3.0, 0.0, 2.0, 1.0]], np.float32)
    ids, w = oracle.route(lg, 3)
    assert ids.tolist() == [[4, 1, 2]]
    s3 = 1 / (1 + math.exp(-3.0))   # 0.9525741268224334
    s2 = 1 / (1 + math.exp(-2.0))   # 0.8807970779778823
    tot = s3 + 2 * s2
    np.testing.assert_array_equal(w[0], np.float32([s3 / tot, s2 / tot, s2 / tot]))
    # all equal logits: the k lowest indices, equal weights
    ids, w = oracle.route(np.zeros((1, 16), np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]]
    assert np.all(w == np.float32(0.25))


def test_route_invariants():
    rng = np.random.default_rng(9)
    lg = (rng.standard_normal((40, 64)) * 4).astype(np.float32)
    for k in (1, 2, 6, 64):
        ids, w = oracle.route(lg, k)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 4 * k * 2 ** -24)
        for r in range(lg.shape[0]):
            assert len(set(ids[r].tolist())) == k
            # slot order: descending logit
            assert np.all(np.diff(lg[r, ids[r]]) <= 0)
        if k == 1:
            assert np.all(w == 1.0)
        if k == 64:
            assert np.all(np.sort(ids, 1) == np.arange(64))


def test_group_matches_stable_sort():
    rng = np.random.default_rng(4)
    for E, A in ((8, 8), (256, 96), (256, 3072)):
        ids = rng.integers(0, E, A).astype(np.int32)
        got = oracle.group(ids, E)
        want = bruteforce.group(ids, E)
        for g, w_ in zip(got, want):
            np.testing.assert_array_equal(g, w_)


def test_group_sentinels_and_invariants():
    ids = np.array([3, -1, 0, 3, -1, 2, 3, 0], np.int32)
    counts, offsets, srt = oracle.group(ids, 4)
    assert counts.tolist() == [2, 0, 1, 3]
    assert offsets.tolist() == [0, 2, 2, 3, 6]
    assert srt.tolist() == [2, 7, 5, 0, 3, 6, -1, -1]
    rng = np.random.default_rng(1)
    ids = rng.integers(-1, 16, 500).astype(np.int32)
    counts, offsets, srt = oracle.group(ids, 16)
    valid = srt[: offsets[-1]]
    assert sorted(valid.tolist()) == [a for a in range(500) if ids[a] >= 0]
    for e in range(16):
        seg = srt[offsets[e]:offsets[e + 1]]
        assert np.all(ids[seg] == e) and np.all(np.diff(seg) > 0)


def test_group_rejects_out_of_range_ids():
    with pytest.raises(ValueError):
        oracle.group(np.array([0, 5], np.int32), 4)
