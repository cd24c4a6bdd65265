"""CPU oracle for the Swin shifted-window multi-head self-attention block forward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP library and imports nothing from it.

Plain float64 numpy, written from the definition of the method, with a library
matmul as the only "primitive".  No blocking, fusion or reordering beyond the
definition: shift, partition, per-window attention, reverse, unshift.

Sources (pages, by title and section):
  * "Boosting Swin Transformer Speed: Profiling, Mixed Precision, and Kernel Fusion
    Secrets" -- Introduction (windowed self-attention with shifted windows),
    Training Optimization (window partition / shift / reverse are index maps;
    fused MHA = QKV GEMM + bias + softmax), Inference Optimization (QKV GEMM with
    bias, invariant data pre-processed once).
  * "Boost Vision Transformer with GPU-Friendly Sparsity and Quantization" --
    Section 3.2 and Figure 3 (the Swin block is the standard transformer block with
    its MHA replaced by shifted-window attention; Q, K, V and output projections
    are GEMMs).
  * "Swin Transformer V2" (research summary) -- How It Works (V1 relative position
    bias; V2 scaled cosine attention with a learnable tau clipped at 0.01 and the
    bias B_ij added; a meta-network on log-spaced relative coordinates gives the
    continuous position bias).
  * "Swin Transformer V2: Scaling Up Capacity and Resolution" -- Abstract (scaled
    cosine attention, log-spaced continuous position bias).

Where the pages are silent the plainest reading is taken; every such reading is
marked "Reading:" below.

Parity pins: every function here is pinned by a ``-m "not gpu"`` test against an
independent formulation (torch's multi-head attention, a dense-mask global
attention, a pure-Python per-token brute force, closed forms, invariants and
hand-derived fixtures).  None is "parity unpinned" against those; against numbers
printed on the pages every function is unpinned, since the pages print none.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Index maps: cyclic shift and window partition (data movement only).
# "Boosting Swin Transformer Speed", Training Optimization: window partition,
# shift and reverse are index-mapping operations.
# ----------------------------------------------------------------------------


def check_geometry(H: int, W: int, M: int, s: int) -> None:
    if M < 1 or H < 1 or W < 1:
        raise ValueError("H, W and M must be positive")
    if H % M or W % M:
        raise ValueError("H and W must be multiples of the window size M")
    if not 0 <= s < M:
        raise ValueError("shift s must satisfy 0 <= s < M")


def cyclic_shift(x: np.ndarray, s: int) -> np.ndarray:
    """Shifted frame of x [B, H, W, C].

    Reading: the map is rolled toward the top-left by s before attention, i.e.
    shifted-frame position (y', x') holds original position ((y'+s) mod H,
    (x'+s) mod W).  The pages name the shift but not its direction.
    """
    _, H, W, _ = x.shape
    ys = (np.arange(H) + s) % H
    xs = (np.arange(W) + s) % W
    return x[:, ys][:, :, xs]


def inverse_cyclic_shift(xs: np.ndarray, s: int) -> np.ndarray:
    """Undo ``cyclic_shift``: original (y, x) holds shifted ((y-s) mod H, (x-s) mod W)."""
    _, H, W, _ = xs.shape
    ys = (np.arange(H) - s) % H
    xx = (np.arange(W) - s) % W
    return xs[:, ys][:, :, xx]


def window_partition(x: np.ndarray, M: int) -> np.ndarray:
    """[B, H, W, C] -> [B*nW, M*M, C]; window w = b*nW + wy*(W/M) + wx,
    in-window token t = ty*M + tx (row-major windows, row-major tokens)."""
    B, H, W, C = x.shape
    t = x.reshape(B, H // M, M, W // M, M, C).transpose(0, 1, 3, 2, 4, 5)
    return t.reshape(B * (H // M) * (W // M), M * M, C)


def window_reverse(xw: np.ndarray, B: int, H: int, W: int, M: int) -> np.ndarray:
    """Inverse of ``window_partition``."""
    C = xw.shape[-1]
    t = xw.reshape(B, H // M, W // M, M, M, C).transpose(0, 1, 3, 2, 4, 5)
    return t.reshape(B, H, W, C)


def partition_shift(x: np.ndarray, M: int, s: int) -> np.ndarray:
    """Cyclic shift then window partition: x [B,H,W,C] -> xw [B*nW, M*M, C]."""
    check_geometry(x.shape[1], x.shape[2], M, s)
    return window_partition(cyclic_shift(x, s), M)


def reverse_unshift(xw: np.ndarray, B: int, H: int, W: int, M: int, s: int) -> np.ndarray:
    """Window reverse then inverse shift: xw [B*nW, M*M, C] -> x [B,H,W,C]."""
    check_geometry(H, W, M, s)
    return inverse_cyclic_shift(window_reverse(xw, B, H, W, M), s)


def window_token_source(B: int, H: int, W: int, M: int, s: int) -> np.ndarray:
    """[B*nW, M*M] flat original-frame token index (b*H*W + y*W + x) held by each
    window slot; partition_shift applied to an iota."""
    iota = np.arange(B * H * W, dtype=np.int64).reshape(B, H, W, 1)
    return partition_shift(iota, M, s)[:, :, 0]


# ----------------------------------------------------------------------------
# Relative position index and shifted-window region mask.
# ----------------------------------------------------------------------------


def relative_position_index(M: int) -> np.ndarray:
    """[N, N] index into a [(2M-1)^2, heads] table for query i, key j.

    "Swin Transformer V2" summary, How It Works: V1 adds a relative position
    bias.  Reading: the offset is coordinate(i) - coordinate(j) in the window,
    row offset major: (ty_i - ty_j + M - 1) * (2M - 1) + (tx_i - tx_j + M - 1).
    """
    t = np.arange(M * M)
    ty, tx = t // M, t % M
    dy = ty[:, None] - ty[None, :] + (M - 1)
    dx = tx[:, None] - tx[None, :] + (M - 1)
    return dy * (2 * M - 1) + dx


def region_labels(H: int, W: int, M: int, s: int) -> np.ndarray:
    """[nW, N] region label of every token of every window (shifted frame).

    Reading (the pages never spell the mask out): along an axis of length L, the
    shifted-frame coordinate v lies in slice 0 if v < L-M, slice 1 if v < L-s,
    else slice 2; the label is 3*slice_y + slice_x.  Two tokens of one window may
    attend to each other only when their labels agree; with s = 0 nothing is
    masked.
    """
    check_geometry(H, W, M, s)
    nW = (H // M) * (W // M)
    if s == 0:
        return np.zeros((nW, M * M), dtype=np.int64)

    def sl(L):
        v = np.arange(L)
        return np.where(v < L - M, 0, np.where(v < L - s, 1, 2))

    lab = 3 * sl(H)[:, None] + sl(W)[None, :]
    return window_partition(lab[None, :, :, None], M)[:, :, 0]


# ----------------------------------------------------------------------------
# V2 continuous position bias.
# "Swin Transformer V2" summary, How It Works: a small meta-network G maps
# relative coordinates to bias values; log-spaced coordinates are used.
# ----------------------------------------------------------------------------


def cpb_log_coords(M: int, coord_scale: float | None = None) -> np.ndarray:
    """[(2M-1)^2, 2] log-spaced (dy, dx) inputs of the meta-network, dy major.

    Reading: u = coord_scale * delta with coord_scale = 8/(M-1) by default, then
    g(u) = sign(u) * log2(1 + |u|) / log2(8) per component.  The log2(8) divisor
    and the factor 8 go together: the window edge maps to log2(9)/3 for every M.
    """
    if coord_scale is None or coord_scale <= 0:
        coord_scale = 8.0 / (M - 1) if M > 1 else 1.0
    d = np.arange(-(M - 1), M, dtype=np.float64)
    dy, dx = np.meshgrid(d, d, indexing="ij")
    u = np.stack([dy.ravel(), dx.ravel()], axis=1) * float(coord_scale)
    return np.sign(u) * np.log2(1.0 + np.abs(u)) / np.log2(8.0)


def cpb_table(w1, b1, w2, b2, M: int, coord_scale: float | None = None) -> np.ndarray:
    """[(2M-1)^2, heads] bias table 16 * sigmoid(W2 relu(W1 g + b1) + b2).

    Reading: hidden width from w1 ([hidden, 2]), ReLU, a second linear layer to
    one value per head ([heads, hidden], bias optional), then 16 * sigmoid.
    """
    g = cpb_log_coords(M, coord_scale)
    hid = np.maximum(g @ np.asarray(w1, np.float64).T + np.asarray(b1, np.float64), 0.0)
    o = hid @ np.asarray(w2, np.float64).T
    if b2 is not None:
        o = o + np.asarray(b2, np.float64)
    return 16.0 / (1.0 + np.exp(-o))


# ----------------------------------------------------------------------------
# The block forward.
# ----------------------------------------------------------------------------


def _attend_windows(xw, region, w_qkv, b_qkv, w_proj, b_proj, bias_table, M, heads,
                    mode, tau, scale, tau_min, eps, masked, want_attn):
    """Attention sub-layer over a batch of windows xw [nw, N, C] (float64)."""
    nw, N, C = xw.shape
    d = C // heads
    # Q, K, V projections are one GEMM with bias ("Boosting Swin Transformer
    # Speed", Inference Optimization; "Boost Vision Transformer...", Figure 3).
    # Reading: nn.Linear layout [3C, C], blocks ordered q | k | v, head h owns
    # channels h*d .. h*d+d-1 of each block.
    qkv = xw @ w_qkv.T + b_qkv
    q = qkv[:, :, 0 * C:1 * C].reshape(nw, N, heads, d).transpose(0, 2, 1, 3)
    k = qkv[:, :, 1 * C:2 * C].reshape(nw, N, heads, d).transpose(0, 2, 1, 3)
    v = qkv[:, :, 2 * C:3 * C].reshape(nw, N, heads, d).transpose(0, 2, 1, 3)
    if mode == "v1":
        # V1: dot-product logits with scale d^-1/2 (reading: the usual MHA scale).
        logits = (q @ k.transpose(0, 1, 3, 2)) * scale
    else:
        # V2: cosine similarity of q and k divided by max(tau, 0.01) ("Swin
        # Transformer V2" summary, How It Works).  Reading: each norm is clamped
        # below at eps before dividing.
        qn = q / np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), eps)
        kn = k / np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), eps)
        t_eff = np.maximum(np.asarray(tau, np.float64), tau_min)
        logits = (qn @ kn.transpose(0, 1, 3, 2)) / t_eff[None, :, None, None]
    rel = relative_position_index(M)
    bias = bias_table[rel.reshape(-1)].reshape(N, N, heads).transpose(2, 0, 1)
    logits = logits + bias[None]
    raw_logits = logits.copy() if want_attn else None
    if masked:
        allowed = region[:, :, None] == region[:, None, :]
        logits = np.where(allowed[:, None], logits, -np.inf)
    # Softmax over the allowed keys, with the row maximum subtracted; disallowed
    # keys get exactly zero weight.
    m = logits.max(axis=-1, keepdims=True)
    p = np.exp(logits - m)
    p = p / p.sum(axis=-1, keepdims=True)
    o = (p @ v).transpose(0, 2, 1, 3).reshape(nw, N, C)
    yw = o @ w_proj.T + b_proj
    return yw, (p if want_attn else None), raw_logits


def wmsa_forward(x, w_qkv, b_qkv, w_proj, b_proj, bias_table, M: int, s: int,
                 heads: int, mode: str = "v1", tau=None, scale: float | None = None,
                 tau_min: float = 0.01, eps: float = 1e-12, windows=None,
                 chunk: int = 32, return_attention: bool = False):
    """Shifted-window MHSA block forward in float64.

    x [B, H, W, C]; w_qkv [3C, C]; b_qkv [3C] or None; w_proj [C, C]; b_proj [C]
    or None; bias_table [(2M-1)^2, heads] (V1 table or V2 CPB table); tau
    [heads] (V2, raw).  Returns y [B, H, W, C].

    With ``windows`` (a sequence of global window indices b*nW + wy*(W/M) + wx)
    only those windows are computed and ``(token_index, y_rows)`` is returned:
    y_rows[i] is the output row of flat original-frame token token_index[i].
    ``return_attention`` (full-window mode only) also returns the attention
    weights [nWin, heads, N, N] and the unmasked logits (bias included).
    """
    x = np.asarray(x, np.float64)
    B, H, W, C = x.shape
    check_geometry(H, W, M, s)
    if C % heads:
        raise ValueError("C must be a multiple of heads")
    d = C // heads
    N = M * M
    nW = (H // M) * (W // M)
    w_qkv = np.asarray(w_qkv, np.float64)
    w_proj = np.asarray(w_proj, np.float64)
    b_qkv = np.zeros(3 * C) if b_qkv is None else np.asarray(b_qkv, np.float64)
    b_proj = np.zeros(C) if b_proj is None else np.asarray(b_proj, np.float64)
    bias_table = np.asarray(bias_table, np.float64)
    if scale is None or scale <= 0:
        scale = d ** -0.5
    if tau_min is None or tau_min <= 0:
        tau_min = 0.01
    if mode not in ("v1", "v2"):
        raise ValueError("mode must be 'v1' or 'v2'")
    if mode == "v2" and tau is None:
        raise ValueError("V2 needs tau")
    region = region_labels(H, W, M, s)
    masked = s > 0
    xw_all = partition_shift(x, M, s)  # [B*nW, N, C]
    sel = np.arange(B * nW) if windows is None else np.asarray(windows, np.int64)
    yw = np.empty((len(sel), N, C))
    attn, logit = [], []
    for c0 in range(0, len(sel), chunk):
        ids = sel[c0:c0 + chunk]
        out, p, lg = _attend_windows(xw_all[ids], region[ids % nW], w_qkv, b_qkv, w_proj,
                                     b_proj, bias_table, M, heads, mode, tau, scale,
                                     tau_min, eps, masked, return_attention)
        yw[c0:c0 + len(ids)] = out
        if return_attention:
            attn.append(p)
            logit.append(lg)
    if windows is not None:
        src = window_token_source(B, H, W, M, s)[sel]
        return src.reshape(-1), yw.reshape(-1, C)
    y = reverse_unshift(yw, B, H, W, M, s)
    if return_attention:
        return y, np.concatenate(attn), np.concatenate(logit)
    return y
