"""CPU oracle for the backward pass of the shifted-window attention sub-layer.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP library and imports nothing from it.

Plain float64 numpy.  Given the forward of ``swin_oracle.wmsa_forward`` and an
upstream gradient dy = dL/dy, it returns dL/d(every input) by the chain rule,
written step by step in the forward's order reversed:

  * "Boosting Swin Transformer Speed", Training Optimization: the fused MHA and
    the index-map (shift / partition) kernels are training speed-ups, so the
    sub-layer is differentiated through the projection, the two attention
    products, the softmax with bias and mask, the QKV projection and the
    transposed index maps.
  * "Swin Transformer V2" summary, How It Works: the V2 logit is the cosine of
    q and k divided by max(tau, 0.01) plus the CPB table entry; the gradient
    reaches tau (where tau > 0.01) and the table.

Readings (the pages are silent on the backward):
  * The gradient of the clamp max(tau, tau_min) is taken as 1 where tau > tau_min
    and 0 where tau <= tau_min; the norm clamp max(|q|, eps) likewise (1 where
    |q| > eps).
  * The table gradient is the sum of dL/dlogit over every (window, query, key)
    pair whose relative position indexes that entry; masked pairs contribute
    nothing (their weight is exactly zero, so is their gradient).
  * The V2 table gradient is with respect to the table the forward consumes
    (the output of the meta-network); ``cpb_backward`` carries it into the
    meta-network's parameters.

Parity pins (``tests/test_oracle_backward.py``): central finite differences of
L = sum(dy * y) through ``swin_oracle.wmsa_forward`` on tiny inputs, for every
input, V1 and V2, with and without the shift; per head and window the table
gradient sums to zero (softmax rows are invariant to a constant added to a
row); the projection-bias gradient is the sum of dy over tokens.
"""
from __future__ import annotations

import numpy as np

from . import swin_oracle as so


def wmsa_backward(x, w_qkv, b_qkv, w_proj, b_proj, bias_table, M: int, s: int, heads: int,
                  dy, mode: str = "v1", tau=None, scale: float | None = None,
                  tau_min: float = 0.01, eps: float = 1e-12, windows=None) -> dict:
    """Gradients of L = sum(dy * wmsa_forward(...)).

    Returns a dict with dx [B,H,W,C], dw_qkv [3C,C], db_qkv [3C], dw_proj [C,C],
    db_proj [C], dtable [(2M-1)^2, heads] and (V2) dtau [heads], all float64.
    V2 also returns dtau_abs [heads]: the same sum over |terms|, which measures
    how far the signed sum cancels (an error scale for dtau, not a gradient).

    windows: optional window indices (0 .. B nW - 1, window order).  Every
    window's part of dx depends only on that window's tokens, so the same
    steps run on those windows alone; the result then holds dxw [len, N, C]
    (the gradient of their slots, mapped to tokens by
    ``swin_oracle.window_token_source``) in place of dx, and the other entries
    sum over those windows only.
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    B, H, W, C = x.shape
    so.check_geometry(H, W, M, s)
    d = C // heads
    N = M * M
    nW = (H // M) * (W // M)
    w_qkv = np.asarray(w_qkv, np.float64)
    w_proj = np.asarray(w_proj, np.float64)
    b_qkv = np.zeros(3 * C) if b_qkv is None else np.asarray(b_qkv, np.float64)
    b_proj = np.zeros(C) if b_proj is None else np.asarray(b_proj, np.float64)
    table = np.asarray(bias_table, np.float64)
    if scale is None or scale <= 0:
        scale = d ** -0.5
    if tau_min is None or tau_min <= 0:
        tau_min = 0.01

    # ---- forward, keeping what the backward needs ------------------------
    xw = so.partition_shift(x, M, s)                      # [nw, N, C]
    widx = np.arange(xw.shape[0]) if windows is None else np.asarray(windows, np.int64)
    xw = xw[widx]
    nw = xw.shape[0]
    qkv = xw @ w_qkv.T + b_qkv
    q = qkv[:, :, 0 * C:1 * C].reshape(nw, N, heads, d).transpose(0, 2, 1, 3)
    k = qkv[:, :, 1 * C:2 * C].reshape(nw, N, heads, d).transpose(0, 2, 1, 3)
    v = qkv[:, :, 2 * C:3 * C].reshape(nw, N, heads, d).transpose(0, 2, 1, 3)
    if mode == "v1":
        sim = q @ k.transpose(0, 1, 3, 2)
        logits = sim * scale
    elif mode == "v2":
        qnorm = np.linalg.norm(q, axis=-1, keepdims=True)
        knorm = np.linalg.norm(k, axis=-1, keepdims=True)
        qn = q / np.maximum(qnorm, eps)
        kn = k / np.maximum(knorm, eps)
        tau = np.asarray(tau, np.float64)
        t_eff = np.maximum(tau, tau_min)
        cos = qn @ kn.transpose(0, 1, 3, 2)
        logits = cos / t_eff[None, :, None, None]
    else:
        raise ValueError("mode must be 'v1' or 'v2'")
    rel = so.relative_position_index(M)
    logits = logits + table[rel.reshape(-1)].reshape(N, N, heads).transpose(2, 0, 1)[None]
    region = so.region_labels(H, W, M, s)
    allowed = np.ones((nw, 1, N, N), bool)
    if s > 0:
        allowed = (region[:, :, None] == region[:, None, :])[widx % nW][:, None]
    logits = np.where(allowed, logits, -np.inf)
    p = np.exp(logits - logits.max(axis=-1, keepdims=True))
    p = p / p.sum(axis=-1, keepdims=True)
    o = (p @ v).transpose(0, 2, 1, 3).reshape(nw, N, C)   # heads concatenated

    # ---- backward ------------------------------------------------------------
    # Output projection y_w = o Wp^T + bp, then the inverse shift: its adjoint is
    # the forward map applied to dy.
    dyw = so.partition_shift(dy, M, s)[widx]              # [nw, N, C]
    db_proj = dyw.sum(axis=(0, 1))
    dw_proj = dyw.reshape(-1, C).T @ o.reshape(-1, C)
    do = (dyw @ w_proj).reshape(nw, N, heads, d).transpose(0, 2, 1, 3)
    # o = p v
    dv = p.transpose(0, 1, 3, 2) @ do
    dp = do @ v.transpose(0, 1, 3, 2)
    # softmax: dlogit = p * (dp - sum_j p dp); zero where masked (p = 0)
    dlogit = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
    # bias: scatter-add into the table rows by relative position
    dtable = np.zeros_like(table)
    g = dlogit.sum(axis=0)                                # [heads, N, N]
    for h in range(heads):
        np.add.at(dtable[:, h], rel.reshape(-1), g[h].reshape(-1))
    out = {}
    if mode == "v1":
        dsim = dlogit * scale
        dq = dsim @ k
        dk = dsim.transpose(0, 1, 3, 2) @ q
    else:
        dcos = dlogit / t_eff[None, :, None, None]
        live = tau > tau_min
        out["dtau"] = np.where(live, -(dlogit * cos).sum(axis=(0, 2, 3)) / t_eff ** 2, 0.0)
        out["dtau_abs"] = np.where(live, np.abs(dlogit * cos).sum(axis=(0, 2, 3)) / t_eff ** 2,
                                   0.0)
        dqn = dcos @ kn
        dkn = dcos.transpose(0, 1, 3, 2) @ qn

        def norm_back(u, un, unorm, dun):
            # un = u / max(|u|, eps): where |u| > eps the Jacobian is
            # (I - un un^T) / |u|, else I / eps.
            big = unorm > eps
            proj = dun - un * (un * dun).sum(axis=-1, keepdims=True)
            return np.where(big, proj / np.maximum(unorm, eps), dun / eps)

        dq = norm_back(q, qn, qnorm, dqn)
        dk = norm_back(k, kn, knorm, dkn)
    dqkv = np.concatenate([t.transpose(0, 2, 1, 3).reshape(nw, N, C) for t in (dq, dk, dv)],
                          axis=-1)                        # [nw, N, 3C]
    db_qkv = dqkv.sum(axis=(0, 1))
    dw_qkv = dqkv.reshape(-1, 3 * C).T @ xw.reshape(-1, C)
    dxw = dqkv @ w_qkv
    out.update(dw_qkv=dw_qkv, db_qkv=db_qkv, dw_proj=dw_proj, db_proj=db_proj, dtable=dtable)
    if windows is not None:
        out["dxw"] = dxw
        return out
    # The forward map's adjoint is the inverse map (a permutation of tokens).
    out["dx"] = so.reverse_unshift(dxw, B, H, W, M, s)
    return out


def cpb_backward(w1, b1, w2, b2, M: int, dtable, coord_scale: float | None = None) -> dict:
    """Gradients of L = sum(dtable * cpb_table(...)) for the meta-network
    parameters: dw1 [hidden, 2], db1 [hidden], dw2 [heads, hidden], db2 [heads]."""
    g = so.cpb_log_coords(M, coord_scale)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    pre = g @ w1.T + np.asarray(b1, np.float64)
    hid = np.maximum(pre, 0.0)
    o = hid @ w2.T
    if b2 is not None:
        o = o + np.asarray(b2, np.float64)
    sig = 1.0 / (1.0 + np.exp(-o))
    do = np.asarray(dtable, np.float64) * 16.0 * sig * (1.0 - sig)
    dw2 = do.T @ hid
    db2 = do.sum(axis=0)
    dpre = (do @ w2) * (pre > 0)
    return {"dw1": dpre.T @ g, "db1": dpre.sum(axis=0), "dw2": dw2, "db2": db2}
