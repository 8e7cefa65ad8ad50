"""Pins of the oracle's top-k selection: brute force on small rows, ties
ordered by index, NaN never selected, short rows padded."""

import itertools

import numpy as np

from oracle import tq_oracle as O


def test_topk_matches_brute_force_sorting():
    rng = np.random.default_rng(0)
    est = rng.standard_normal((20, 37))
    idx, vals = O.topk(est, 7)
    for r in range(20):
        ranked = sorted(range(37), key=lambda j: (-est[r, j], j))[:7]
        assert list(idx[r]) == ranked
        assert np.array_equal(vals[r], est[r, ranked])


def test_topk_ties_go_to_smaller_index_and_nan_is_skipped():
    est = np.array([[1.0, 3.0, 3.0, np.nan, 2.0, 3.0]])
    idx, vals = O.topk(est, 4)
    assert list(idx[0]) == [1, 2, 5, 4]
    assert list(vals[0]) == [3.0, 3.0, 3.0, 2.0]


def test_topk_short_rows_are_padded():
    idx, vals = O.topk(np.array([[0.5, -1.0], [np.nan, np.nan]]), 3)
    assert list(idx[0]) == [0, 1, -1] and vals[0, 2] == -np.inf
    assert list(idx[1]) == [-1, -1, -1]


def test_topk_every_permutation_of_a_small_row():
    base = np.array([0.1, 0.7, 0.7, -0.2])
    for perm in itertools.permutations(range(4)):
        row = base[list(perm)]
        idx, _ = O.topk(row[None, :], 2)
        best = [j for j in range(4) if row[j] == 0.7]
        assert list(idx[0]) == sorted(best)
