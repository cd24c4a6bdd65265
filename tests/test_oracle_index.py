"""Pins of the oracle's index maps (cyclic shift, window partition, relative index,
region mask) against hand-derived fixtures, closed forms and a second formulation.
CPU only."""
import json
import os

import numpy as np
import pytest

from oracle import bruteforce, swin_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

GEOMS = [  # (B, H, W, M, s)
    (1, 4, 4, 2, 1), (2, 6, 6, 3, 1), (1, 8, 12, 4, 2), (2, 14, 14, 7, 3),
    (1, 7, 7, 7, 3), (1, 16, 16, 16, 8), (3, 6, 9, 3, 0), (1, 5, 5, 1, 0),
]


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("B,H,W,M,s", GEOMS)
def test_partition_reverse_identity_bits(B, H, W, M, s):
    rng = np.random.default_rng(7)
    x = rng.integers(-2**15, 2**15, size=(B, H, W, 5), dtype=np.int16)
    xw = so.partition_shift(x, M, s)
    assert xw.shape == (B * (H // M) * (W // M), M * M, 5)
    back = so.reverse_unshift(xw, B, H, W, M, s)
    assert np.array_equal(back, x)
    # shift and unshift alone are identities too
    assert np.array_equal(so.inverse_cyclic_shift(so.cyclic_shift(x, s), s), x)
    assert np.array_equal(so.window_reverse(so.window_partition(x, M), B, H, W, M), x)


@pytest.mark.parametrize("B,H,W,M,s", GEOMS)
def test_partition_iota_closed_form(B, H, W, M, s):
    """Every window slot holds the source token given by the closed form, written
    here with explicit loops; every source token appears exactly once."""
    src = so.window_token_source(B, H, W, M, s)
    nWx = W // M
    nW = (H // M) * nWx
    for w in range(B * nW):
        b, r = divmod(w, nW)
        wy, wx = divmod(r, nWx)
        for t in range(M * M):
            ty, tx = divmod(t, M)
            y = (wy * M + ty + s) % H
            x = (wx * M + tx + s) % W
            assert src[w, t] == (b * H + y) * W + x
    assert np.array_equal(np.sort(src.ravel()), np.arange(B * H * W))


def test_relative_index_golden():
    g = _golden("rel_index_M2.json")
    assert np.array_equal(so.relative_position_index(g["M"]), np.array(g["index"]))


@pytest.mark.parametrize("M", [1, 2, 3, 7, 16, 24])
def test_relative_index_properties(M):
    idx = so.relative_position_index(M)
    n = M * M
    centre = (M - 1) * (2 * M - 1) + (M - 1)
    assert np.all(np.diag(idx) == centre)
    assert idx.min() >= 0 and idx.max() == (2 * M - 1) ** 2 - 1
    # antisymmetry of the offset: idx(i,j) + idx(j,i) = 2 * centre
    assert np.all(idx + idx.T == 2 * centre)
    assert idx.shape == (n, n)


def test_region_golden():
    g = _golden("region_H4_W4_M2_s1.json")
    H, W, M, s = g["H"], g["W"], g["M"], g["s"]
    lab = so.region_labels(H, W, M, s)
    expect = so.window_partition(np.array(g["labels_shifted_frame"])[None, :, :, None], M)[:, :, 0]
    assert np.array_equal(lab, expect)
    for w, groups in g["groups_per_window_tokens"].items():
        w = int(w)
        for grp in groups:
            assert len({lab[w, t] for t in grp}) == 1
        reps = [lab[w, grp[0]] for grp in groups]
        assert len(set(reps)) == len(reps)


def _mask_from_labels(B, H, W, M, s):
    lab = so.region_labels(H, W, M, s)
    src = so.window_token_source(1, H, W, M, s)
    pairs = set()
    for w in range(lab.shape[0]):
        for i in range(M * M):
            for j in range(M * M):
                if lab[w, i] == lab[w, j]:
                    yi, xi = divmod(int(src[w, i]), W)
                    yj, xj = divmod(int(src[w, j]), W)
                    pairs.add(((yi, xi), (yj, xj)))
    return pairs


CASES_MASK = [(H, W, M, s) for M in range(2, 6) for s in range(0, M)
              for (H, W) in [(M, M), (2 * M, M), (2 * M, 3 * M)]]


@pytest.mark.parametrize("H,W,M,s", CASES_MASK)
def test_region_mask_equals_no_wrap_rule(H, W, M, s):
    """The slice-label mask and the no-wrap formulation agree pair for pair."""
    assert _mask_from_labels(1, H, W, M, s) == bruteforce.allowed_pairs(H, W, M, s)


def test_region_counts_swin_shapes():
    """Masked windows per image: only the last window row and column mix slices."""
    for (H, M, s, masked) in [(56, 7, 3, 15), (14, 7, 3, 3), (64, 16, 8, 7), (384, 24, 12, 31)]:
        lab = so.region_labels(H, H, M, s)
        n = sum(len(set(row.tolist())) > 1 for row in lab)
        assert n == masked
    assert np.all(so.region_labels(56, 56, 7, 0) == 0)
