"""Pins of the 2:4 sparsity oracle (oracle/swin_sparse.py): the pruning rule by
brute force, the compressed form's round trip, idempotence, and the layer as
explicit loops."""
import itertools

import numpy as np

from oracle import swin_sparse as sp

RNG = np.random.default_rng(21)


def test_prune_keeps_two_largest_per_group():
    w = RNG.normal(size=(7, 32))
    p = sp.prune24(w)
    for r in range(7):
        for g in range(8):
            grp, kept = w[r, 4 * g:4 * g + 4], p[r, 4 * g:4 * g + 4]
            assert np.count_nonzero(kept) == 2
            # Brute force over the six pairs: the kept pair has the largest |sum|.
            best = max(itertools.combinations(range(4), 2),
                       key=lambda c: (abs(grp[c[0]]) + abs(grp[c[1]]), -c[0], -c[1]))
            assert set(np.flatnonzero(kept)) == set(best)
            np.testing.assert_array_equal(kept[list(best)], grp[list(best)])


def test_ties_keep_lower_positions():
    w = np.array([[1.0, -1.0, 1.0, 1.0, 0.0, 0.0, 0.0, 5.0]])
    np.testing.assert_array_equal(sp.prune24(w), [[1.0, -1.0, 0, 0, 0, 0, 0, 5.0]])


def test_compress_round_trip_and_idempotence():
    w = sp.prune24(RNG.normal(size=(5, 64)))
    vals, codes = sp.compress24(w)
    assert vals.shape == (5, 32) and codes.shape == (5, 16)
    np.testing.assert_array_equal(sp.expand24(vals, codes, 64), w)
    np.testing.assert_array_equal(sp.prune24(w), w)
    p0, p1 = codes & 3, codes >> 2
    assert np.all(p0 < p1)


def test_layer_equals_loops():
    x = RNG.normal(size=(3, 16))
    wp = sp.prune24(RNG.normal(size=(4, 16)))
    b = RNG.normal(size=4)
    y = sp.linear_sparse24(x, wp, b)
    for t in range(3):
        for n in range(4):
            s = b[n] + sum(x[t, k] * wp[n, k] for k in range(16))
            assert abs(y[t, n] - s) < 1e-12
