"""Per-token brute-force shifted-window attention, pure Python (tiny inputs only).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only ``tests/`` use it.

It shares no step with ``swin_oracle.wmsa_forward``: no roll, no partition, no
region labels.  Each output token is computed directly in the original frame:

  * token p = (y, x) sits at shifted-frame position ((y - s) mod H, (x - s) mod W)
    (the oracle's shift-direction reading);
  * p' is a key of p iff both fall in the same shifted-frame window AND the
    shifted-frame offset equals the original-frame offset on both axes, i.e. no
    wrap-around of the cyclic shift lies between them (the other formulation of
    the shifted-window mask: tokens that were only brought next to each other by
    the wrap may not attend to each other);
  * the relative-position bias is looked up with the shifted-frame offset,
    table row (dy + M - 1) * (2M - 1) + (dx + M - 1).

Pages: "Boosting Swin Transformer Speed" (Introduction: shifted windows);
"Swin Transformer V2" summary (How It Works: relative position bias, scaled cosine
attention with tau clipped at 0.01).
"""
from __future__ import annotations

import math


def _linear(w, b, v):
    return [sum(w[o][i] * v[i] for i in range(len(v))) + (b[o] if b is not None else 0.0)
            for o in range(len(w))]


def _keys_of(H, W, M, s, y, xx):
    """Original-frame keys (y2, x2, dy, dx) that token (y, xx) attends to; (dy, dx)
    is the shifted-frame offset query minus key."""
    ys, xs = (y - s) % H, (xx - s) % W
    keys = []
    for y2 in range(H):
        for x2 in range(W):
            y2s, x2s = (y2 - s) % H, (x2 - s) % W
            if y2s // M != ys // M or x2s // M != xs // M:
                continue
            if (ys - y2s) != (y - y2) or (xs - x2s) != (xx - x2):
                continue
            keys.append((y2, x2, ys - y2s, xs - x2s))
    return keys


def wmsa_forward(x, w_qkv, b_qkv, w_proj, b_proj, table, M, s, heads, mode, tau=None,
                 scale=None, tau_min=0.01):
    """All output tokens as nested lists [B][H][W][C].  Inputs are nested lists or
    arrays indexable as x[b][y][x][c]; float64 (Python float) arithmetic."""
    B, H, W, C = len(x), len(x[0]), len(x[0][0]), len(x[0][0][0])
    d = C // heads
    if scale is None:
        scale = d ** -0.5
    w_qkv = [[float(a) for a in row] for row in w_qkv]
    w_proj = [[float(a) for a in row] for row in w_proj]
    b_qkv = None if b_qkv is None else [float(a) for a in b_qkv]
    b_proj = None if b_proj is None else [float(a) for a in b_proj]
    out = []
    for b in range(B):
        qkv = {(yy, xv): _linear(w_qkv, b_qkv, [float(c) for c in x[b][yy][xv]])
               for yy in range(H) for xv in range(W)}
        img = []
        for yy in range(H):
            row = []
            for xv in range(W):
                keys = _keys_of(H, W, M, s, yy, xv)
                o = [0.0] * C
                for h in range(heads):
                    q = qkv[(yy, xv)][h * d:(h + 1) * d]
                    logits, vals = [], []
                    for (y2, x2, dy, dx) in keys:
                        kv = qkv[(y2, x2)]
                        k = kv[C + h * d:C + (h + 1) * d]
                        dot = sum(q[c] * k[c] for c in range(d))
                        if mode == "v1":
                            lg = scale * dot
                        else:
                            nq = max(math.sqrt(sum(c * c for c in q)), 1e-12)
                            nk = max(math.sqrt(sum(c * c for c in k)), 1e-12)
                            lg = dot / (nq * nk) / max(float(tau[h]), tau_min)
                        lg += float(table[(dy + M - 1) * (2 * M - 1) + (dx + M - 1)][h])
                        logits.append(lg)
                        vals.append(kv[2 * C + h * d:2 * C + (h + 1) * d])
                    mx = max(logits)
                    e = [math.exp(l - mx) for l in logits]
                    z = sum(e)
                    for c in range(d):
                        o[h * d + c] = sum(e[j] * vals[j][c] for j in range(len(e))) / z
                row.append(_linear(w_proj, b_proj, o))
            img.append(row)
        out.append(img)
    return out


def allowed_pairs(H, W, M, s):
    """Set of ((y, x), (y2, x2)) original-frame pairs that may attend (any image)."""
    out = set()
    for y in range(H):
        for x in range(W):
            ys, xs = (y - s) % H, (x - s) % W
            for y2 in range(H):
                for x2 in range(W):
                    y2s, x2s = (y2 - s) % H, (x2 - s) % W
                    if y2s // M == ys // M and x2s // M == xs // M and \
                            ys - y2s == y - y2 and xs - x2s == x - x2:
                        out.add(((y, x), (y2, x2)))
    return out
