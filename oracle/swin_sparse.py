"""CPU oracle for 2:4 structured-sparse QKV / projection linear layers.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP library and imports nothing from it.

"Boost Vision Transformer with GPU-Friendly Sparsity and Quantization", Section
3.1 and Figure 1: 2:4 fine-grained structured sparsity keeps two of every four
consecutive weights along the reduction (input-channel) dimension and stores
the kept values with their positions, which the sparse matrix cores consume at
twice the dense rate; Section 3.2 / Figure 3 applies it to the QKV, projection
and feed-forward GEMMs of each block.
Readings (the pages leave these open):
  * The pruning rule: in each group of four along K the two of largest
    magnitude are kept (ties: the lower position), which is the plain
    magnitude criterion; trained 2:4 weights are out of scope, so the layers
    run on seeded weights pruned this way.
  * Compressed form: per row, the kept values in group order (two per group,
    the lower position first) and, per group, the two positions (2 bits each,
    the first in bits 0-1, the second in bits 2-3).
  * y = x wp^T + bias with wp the pruned dense matrix, exactly (float64).

Parity pins (``tests/test_oracle_sparse.py``): exactly two nonzeros per group,
the kept ones are the two largest, compress / expand round trip, a matrix
that already is 2:4 is unchanged, and the layer equals the dense product with
the pruned matrix computed by loops.
"""
from __future__ import annotations

import numpy as np


def prune24(w) -> np.ndarray:
    """Dense copy of w [N, K] (K % 4 == 0) with the two smallest-magnitude
    entries of every group of four along K set to zero."""
    w = np.asarray(w, np.float64)
    N, K = w.shape
    g = w.reshape(N, K // 4, 4)
    # Stable sort by descending magnitude: ties keep the lower position first.
    order = np.argsort(-np.abs(g), axis=-1, kind="stable")
    keep = np.zeros_like(g, dtype=bool)
    np.put_along_axis(keep, order[..., :2], True, axis=-1)
    return np.where(keep, g, 0.0).reshape(N, K)


def compress24(wp) -> tuple[np.ndarray, np.ndarray]:
    """(values [N, K/2], positions [N, K/4] uint8 = p0 | p1 << 2) of a 2:4 matrix
    (exactly two kept entries per group, zeros counted as kept where a group has
    fewer than two nonzeros: the lowest free positions fill it)."""
    wp = np.asarray(wp, np.float64)
    N, K = wp.shape
    g = wp.reshape(N, K // 4, 4)
    nz = g != 0
    # Positions: the nonzeros in order, then zero positions in order, first two.
    key = np.where(nz, 0, 1) * 4 + np.arange(4)
    pos = np.sort(np.argsort(key, axis=-1, kind="stable")[..., :2], axis=-1)
    vals = np.take_along_axis(g, pos, axis=-1)
    codes = (pos[..., 0] | (pos[..., 1] << 2)).astype(np.uint8)
    return vals.reshape(N, K // 2), codes


def expand24(vals, codes, K: int) -> np.ndarray:
    vals = np.asarray(vals, np.float64)
    codes = np.asarray(codes, np.int64)
    N = vals.shape[0]
    out = np.zeros((N, K // 4, 4))
    v = vals.reshape(N, K // 4, 2)
    p0, p1 = codes & 3, (codes >> 2) & 3
    np.put_along_axis(out, p0[..., None], v[..., :1], axis=-1)
    np.put_along_axis(out, p1[..., None], v[..., 1:], axis=-1)
    return out.reshape(N, K)


def linear_sparse24(x, wp, bias=None) -> np.ndarray:
    y = np.asarray(x, np.float64) @ np.asarray(wp, np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)
    return y
